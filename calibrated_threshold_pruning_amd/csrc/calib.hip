// Threshold calibration for bfloat16 inputs on gfx950 ("Top-Theta Attention:
// Sparsifying Transformers by Compensated Thresholding", Sec. 3.1, Algorithm 1,
// in its post-softmax form): for every calibration sequence, head and query
// row p, the k-th largest post-softmax value of the causal row (keys 0..p),
// for up to eight targets k at once.  A sample is the k-th largest score x_k
// (log2 domain) turned into exp2(x_k - lse2), lse2 = log2 of the row's
// softmax denominator.
//
// Workgroup (1024 threads): C score columns, each one (head, query row) of a
// single sequence and KV group.  Phase 1 forms the C causal score rows on MFMA
// (K rows as the A operand, the C query rows as the columns of the B operand)
// into LDS; alongside, every lane keeps the running maximum, softmax sum and
// score sum of its column (the exp work overlaps the K loads).  Phase 2 gives
// each column 1024 / C threads:
//   * a histogram of (m - x), m the row maximum, in NB bins over a window of
//     twice the distance from m to the mean score (the last bin open-ended);
//     binning is monotone in x, so the bin holding the k-th largest and the
//     rank inside it follow from one prefix scan, for every k;
//   * the members of that bin are copied out and the exact value is found by
//     counting, among them, the values above and at each member;
//   * a bin with more members than the copy space holds (long runs of equal
//     scores, or a k-th largest beyond the window) is resolved by a radix
//     select (8-bit digits of the order-preserving 32-bit key) restricted to
//     the bin.
// Samples go to a [S][n_k][Hq][Lq] buffer and are summed over the sequences
// in a fixed order afterwards.
//
// Pre-softmax form (Algorithm 1 as printed): the sample is the k-th largest
// score itself, in score units; optionally also the discarded mass of the
// row's top-k relative to the row maximum (the offline estimate of E~ in
// Sec. 3.2.1), from one more pass over the column's scores.
#include "topth_internal.h"

#include <type_traits>

#include <math.h>

namespace topth {

constexpr int kCalThreads = 1024;
constexpr int kCalWaves = kCalThreads / 64;
constexpr int kCalHistWords = 4096;    // histogram words per workgroup (all columns)

struct CalibKArgs {
    const uint16_t* q; const uint16_t* k;
    int S, Hq, Hkv, Lq, Lk, q_pos0;
    int nks;            // LDS stride of a score column (floats, multiple of 4)
    int gh, rb;         // heads x rows per workgroup (gh * rb = C)
    int nblk, ngh;      // row blocks per head, head groups per sequence
    unsigned nwg;       // workgroups in the grid (nblk * ngh * S)
    float xscale;       // scale * log2(e)
    int ks[8]; int n_k;
    float* samples;     // [S][n_k][Hq][Lq]
    float* esamples;    // pre-softmax: discarded mass of the top-k, same shape, or NULL
    int pre;            // 1: samples are k-th largest scores (pre-softmax)
};

template <int C>
struct CalCfg {
    static constexpr int TPC = kCalThreads / C;     // threads per column (>= 64)
    static constexpr int WPC = TPC / 64;            // waves per column
    static constexpr int NB = kCalHistWords / C;    // bins per column
    static constexpr int BPT = NB / TPC;            // bins per thread in the scan (4)
    static_assert(BPT * TPC == NB, "bins must split evenly over a column's threads");
};

// Exclusive prefix sum of v over the threads of one column, in thread order.
// A column's waves are consecutive: one wave-level scan, then a cross-wave
// step through LDS.  Every thread of the workgroup must call it (it holds
// barriers when a column spans several waves).
template <int WPC>
__device__ __forceinline__ int col_exscan(int v, int* red) {
    const int lane = threadIdx.x & 63;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    int off = 0;
    if constexpr (WPC > 1) {
        const int wave = threadIdx.x >> 6;
        if (lane == 63) red[wave] = x;
        __syncthreads();
        for (int i = wave / WPC * WPC; i < wave; ++i) off += red[i];
        __syncthreads();
    }
    return x - v + off;
}

// Sum of v over the threads of one column, added in a fixed order (every
// thread of the workgroup must call it; every thread of the column gets it).
template <int WPC>
__device__ __forceinline__ float col_sum(float v, float* red) {
    float x = wave_sum(v);
    if constexpr (WPC > 1) {
        const int wave = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) red[wave] = x;
        __syncthreads();
        x = 0.f;
        for (int i = wave / WPC * WPC; i < wave / WPC * WPC + WPC; ++i) x += red[i];
        __syncthreads();
    }
    return x;
}

// bin of score x in a column with maximum m: bins of 1/bs log2 units below m,
// the last bin open-ended; monotone non-increasing in x
template <int NB>
__device__ __forceinline__ int score_bin(float m, float bs, float x) {
    const float d = (m - x) * bs;
    return d < (float)(NB - 1) ? (int)d : NB - 1;
}

// merge two (max, sum of exp2(x - max)) pairs
__device__ __forceinline__ void merge_ms(float& m, float& s, float m2, float s2) {
    const float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;
    s = s * __builtin_amdgcn_exp2f(m - mn) + s2 * __builtin_amdgcn_exp2f(m2 - mn);
    m = mn;
}

template <int D, int C>
__global__ __launch_bounds__(kCalThreads) void calib_bf16_kernel(CalibKArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)   // the host pass only needs the launch stub
    using G = CalCfg<C>;
    constexpr int TPC = G::TPC, WPC = G::WPC, NB = G::NB, BPT = G::BPT;
    constexpr int KSTEPS = D / 32;
    extern __shared__ __attribute__((aligned(16))) float xs[];      // [C][nks] scores
    uint32_t* hist = reinterpret_cast<uint32_t*>(xs + C * a.nks);   // [C][NB]
    __shared__ float s_stat[kCalWaves][16][3];                      // per wave: max, sum, score sum
    __shared__ int redi[kCalWaves];
    __shared__ float redf[kCalWaves];
    __shared__ int s_bin[C][8], s_rank[C][8], s_cnt[C][8], s_fill[C][8];
    __shared__ float s_val[C][8];
    __shared__ int s_dig[C], s_kk[C];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    // XCD-aware order: workgroup b runs on XCD b % 8; consecutive workgroups of
    // one XCD take consecutive row blocks of one (sequence, head group), so a
    // sequence's K rows are fetched into one XCD's L2 and reused there
    unsigned wg = blockIdx.x;
    {
        const unsigned per = a.nwg / 8u;
        if (wg < 8u * per) wg = (wg & 7u) * per + (wg >> 3);
    }
    const int rblk = (int)(wg % (unsigned)a.nblk);
    const int hg = (int)((wg / (unsigned)a.nblk) % (unsigned)a.ngh);
    const int s = (int)(wg / ((unsigned)a.nblk * (unsigned)a.ngh));
    const int i0 = (a.nblk - 1 - rblk) * a.rb;            // longest rows first
    const int h0 = hg * a.gh;
    const int kv = h0 / (a.Hq / a.Hkv);
    const int nkeys = a.q_pos0 + min(i0 + a.rb, a.Lq);      // keys seen by the block's last row

    // column of this thread in phase 2
    const int c = tid / TPC, u = tid % TPC;
    uint32_t* hc = hist + c * NB;
    if (u < 8) { s_bin[c][u] = -1; s_fill[c][u] = 0; s_cnt[c][u] = 0; s_rank[c][u] = 0; }
    for (int i = u; i < NB; i += TPC) hc[i] = 0u;

    // ---- phase 1: S^T = K Q^T on MFMA (keys in the 16 A rows, columns in B);
    // scores to LDS, and per lane the running max, softmax sum and score sum of
    // its column over the causal keys
    {
        const int l16 = lane & 15, lq = lane >> 4;
        bf16x8 qf[KSTEPS];
        const int ii = i0 + l16 % a.rb, hh = h0 + l16 / a.rb;
        const bool ok = l16 < C && ii < a.Lq;
        const int ncol = ok ? a.q_pos0 + ii + 1 : 0;
        const uint16_t* qr = a.q + (((size_t)s * a.Hq + (ok ? hh : 0)) * a.Lq + (ok ? ii : 0)) * D;
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st) {
            const u32x4 raw = *(const u32x4*)(qr + 32 * st + 8 * lq);
            const u32x4 z = {0u, 0u, 0u, 0u};
            qf[st] = __builtin_bit_cast(bf16x8, ok ? raw : z);
        }
        const uint16_t* kg = a.k + ((size_t)s * a.Hkv + kv) * (size_t)a.Lk * D + 8 * lq;
        const int ntile = (nkeys + 15) / 16;
        float mloc = -INFINITY, sloc = 0.f, xsum = 0.f;
        auto kload = [&](u32x4 (&dst)[KSTEPS], int t) {
            const uint16_t* kr = kg + (size_t)min(16 * t + l16, nkeys - 1) * D;
#pragma unroll
            for (int st = 0; st < KSTEPS; ++st) dst[st] = *(const u32x4*)(kr + 32 * st);
        };
        // every live column of the block sees at least the keys of its first row
        const int nfull = a.q_pos0 + i0 + 1;
        auto kuse = [&](const u32x4 (&src)[KSTEPS], int t) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < KSTEPS; ++st)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, src[st]), qf[st],
                                                               acc, 0, 0, 0);
            f32x4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = acc[r] * a.xscale;
            if (16 * t + 16 <= nfull) {            // whole tile inside every live column (wave-uniform)
                if (l16 < C) *(f32x4*)(xs + l16 * a.nks + 16 * t + 4 * lq) = v;
                const float tmax = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
                if (tmax > mloc) { sloc *= __builtin_amdgcn_exp2f(mloc - tmax); mloc = tmax; }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sloc += __builtin_amdgcn_exp2f(v[r] - mloc);
                    xsum += v[r];
                }
            } else {                               // keys past a column's row are stored as -inf
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (16 * t + 4 * lq + r >= ncol) v[r] = -INFINITY;
                if (l16 < C) *(f32x4*)(xs + l16 * a.nks + 16 * t + 4 * lq) = v;
                const float tmax = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
                if (tmax > mloc) { sloc *= __builtin_amdgcn_exp2f(mloc - tmax); mloc = tmax; }
                if (mloc > -INFINITY) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        sloc += __builtin_amdgcn_exp2f(v[r] - mloc);
                        xsum += v[r] > -INFINITY ? v[r] : 0.f;
                    }
                }
            }
        };
        // three K tiles per wave in flight: the one in use and the next two
        u32x4 ka[KSTEPS], kb[KSTEPS], kc[KSTEPS];
        int t = wave;
        if (t < ntile) kload(ka, t);
        if (t + kCalWaves < ntile) kload(kb, t + kCalWaves);
        while (t < ntile) {
            if (t + 2 * kCalWaves < ntile) kload(kc, t + 2 * kCalWaves);
            kuse(ka, t);
            t += kCalWaves;
            if (t >= ntile) break;
            if (t + 2 * kCalWaves < ntile) kload(ka, t + 2 * kCalWaves);
            kuse(kb, t);
            t += kCalWaves;
            if (t >= ntile) break;
            if (t + 2 * kCalWaves < ntile) kload(kb, t + 2 * kCalWaves);
            kuse(kc, t);
            t += kCalWaves;
        }
        // four -inf past the last tile: phase 2 reads whole float4 groups up to a row's end
        if (wave == 0 && lq == 0 && l16 < C) {
            const f32x4 ninf = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            *(f32x4*)(xs + l16 * a.nks + 16 * ntile) = ninf;
        }
        // lanes l16, l16+16, l16+32, l16+48 hold the same column
#pragma unroll
        for (int o = 16; o < 64; o <<= 1) {
            const float m2 = __shfl_xor(mloc, o), s2 = __shfl_xor(sloc, o);
            xsum += __shfl_xor(xsum, o);
            merge_ms(mloc, sloc, m2, s2);
        }
        if (lane < 16) { s_stat[wave][lane][0] = mloc; s_stat[wave][lane][1] = sloc; s_stat[wave][lane][2] = xsum; }
    }
    __syncthreads();

    // ---- phase 2: per column
    const int ii = i0 + c % a.rb, hh = h0 + c / a.rb;
    const bool live = ii < a.Lq;
    const int n = live ? a.q_pos0 + ii + 1 : 0;              // causal row length
    const float* xr = xs + c * a.nks;

    // column statistics, merged over the waves in a fixed order
    float m = -INFINITY, l = 0.f, xsum = 0.f;
    for (int w = 0; w < kCalWaves; ++w) {
        merge_ms(m, l, s_stat[w][c][0], s_stat[w][c][1]);
        xsum += s_stat[w][c][2];
    }
    const float lse2 = m + log2f(l);
    // histogram window: twice the distance from the maximum to the mean score
    const float width = live ? fmaxf(2.0f * (m - xsum / (float)n), 1.0f / 64.0f) : 1.0f;
    const float bs = (float)NB / width;

    // whole float4 groups: the up to three -inf past the row end land in the
    // last bin and are taken out again below
    for (int j = 4 * u; j < n; j += 4 * TPC) {
        const f32x4 v = *(const f32x4*)(xr + j);
#pragma unroll
        for (int e = 0; e < 4; ++e) atomicAdd(&hc[score_bin<NB>(m, bs, v[e])], 1u);
    }
    __syncthreads();

    // bin and in-bin rank of the k-th largest, for every k
    {
        int hv[BPT], local = 0;
#pragma unroll
        for (int e = 0; e < BPT; ++e) hv[e] = (int)hc[BPT * u + e];
        if (u == TPC - 1) hv[BPT - 1] -= ((n + 3) & ~3) - n;    // bin NB - 1
#pragma unroll
        for (int e = 0; e < BPT; ++e) local += hv[e];
        const int pre = col_exscan<WPC>(local, redi);
        for (int t = 0; t < a.n_k; ++t) {
            const int kk = a.ks[t];
            if (n > kk && pre < kk && kk <= pre + local) {
                int cum = pre;
#pragma unroll
                for (int e = 0; e < BPT; ++e) {
                    if (cum < kk && kk <= cum + hv[e]) {
                        s_bin[c][t] = BPT * u + e;
                        s_rank[c][t] = kk - cum;
                        s_cnt[c][t] = hv[e];
                    }
                    cum += hv[e];
                }
            }
        }
    }
    __syncthreads();

    // copy out the members of each target bin (the histogram space is reused)
    const int cap = NB / a.n_k;
    float* cand = reinterpret_cast<float*>(hc);
    int tb[8];
    int bmin = NB, bmax = -1;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        // members of the open-ended last bin are left to the radix path
        tb[t] = (t < a.n_k && s_cnt[c][t] <= cap && s_bin[c][t] < NB - 1) ? s_bin[c][t] : -1;
        if (tb[t] >= 0) { bmin = min(bmin, tb[t]); bmax = max(bmax, tb[t]); }
    }
    // slots: per wave, a ballot of the lanes holding a member and their rank in
    // it; a column of one wave keeps the running count in registers, wider
    // columns reserve space with one atomic per wave
    int run[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) run[t] = 0;
    const int jend = __builtin_amdgcn_readfirstlane(n);
    for (int j0 = 4 * (u - lane); j0 < jend; j0 += 4 * TPC) {   // uniform per wave
        const int j = j0 + 4 * lane;
        const f32x4 v = *(const f32x4*)(xr + j);
        const bool jok = j < n;                // the -inf past the row end fall outside the range
        const float dlo = (float)bmin, dhi = (float)(bmax + 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float dd = (m - v[e]) * bs;  // bin = floor(dd) inside the range (all below NB - 1)
            const bool in = jok && dd >= dlo && dd < dhi;
            const int b = (int)dd;
            if (!__builtin_amdgcn_ballot_w64(in)) continue;      // uniform
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                if (t >= a.n_k) break;
                const bool hit = in && b == tb[t];
                const unsigned long long bal = __builtin_amdgcn_ballot_w64(hit);
                if (!bal) continue;
                const int cntw = __popcll(bal);
                int base;
                if constexpr (WPC == 1) {
                    base = run[t];
                    run[t] += cntw;
                } else {
                    const int leader = __ffsll((long long)bal) - 1;
                    int b0 = 0;
                    if (lane == leader) b0 = atomicAdd(&s_fill[c][t], cntw);
                    base = __builtin_amdgcn_readlane(b0, leader);
                }
                const int slot = base + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32),
                                                                       __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
                if (hit && slot < cap) cand[t * cap + slot] = v[e];
            }
        }
    }
    __syncthreads();

    // exact value inside each copied bin: the member with (#greater < rank <= #greater-or-equal)
    for (int t = 0; t < a.n_k; ++t) {
        if (tb[t] < 0) continue;
        const int cnt = __builtin_amdgcn_readfirstlane(s_cnt[c][t]);
        const int rank = s_rank[c][t];
        const float* cb = cand + t * cap;
        if (cnt <= 64) {
            if (u < 64) {                  // the column's first wave, members in its lanes
                const float x = u < cnt ? cb[u] : -INFINITY;
                int gt = 0, ge = 0;
                for (int j = 0; j < cnt; ++j) {
                    const float y = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), j));
                    gt += y > x;
                    ge += y >= x;
                }
                if (u < cnt && gt < rank && rank <= ge) s_val[c][t] = x;   // equal members agree
            }
        } else {
            for (int i = u; i < cnt; i += TPC) {
                const float x = cb[i];
                int gt = 0, ge = 0;
                for (int j = 0; j < cnt; ++j) {
                    const float y = cb[j];
                    gt += y > x;
                    ge += y >= x;
                }
                if (gt < rank && rank <= ge) s_val[c][t] = x;
            }
        }
    }

    // crowded bins: radix select over the order-preserving keys of the bin's members
    bool crowded = false;
    for (int t = 0; t < a.n_k; ++t) crowded |= s_bin[c][t] >= 0 && tb[t] < 0;
    if (__syncthreads_or(crowded)) {
        constexpr int DPT = TPC >= 256 ? 1 : 256 / TPC;     // digits per thread in the scan
        for (int t = 0; t < a.n_k; ++t) {
            const int bin = s_bin[c][t];
            const bool want = bin >= 0 && tb[t] < 0;
            uint32_t prefix = 0u, mask = 0u;
            int kk = s_rank[c][t];
            for (int shift = 24; shift >= 0; shift -= 8) {
                for (int i = u; i < 256; i += TPC) hc[i] = 0u;
                __syncthreads();
                if (want)
                    for (int j = u; j < n; j += TPC) {
                        const float x = xr[j];
                        if (score_bin<NB>(m, bs, x) != bin) continue;
                        const uint32_t key = float_to_ordered(x);
                        if ((key & mask) == prefix) atomicAdd(&hc[(key >> shift) & 255u], 1u);
                    }
                __syncthreads();
                // digits from the top: thread u holds digits top, top-1, ..., top-DPT+1
                const int top = 255 - u * DPT;
                int dv[DPT], local = 0;
#pragma unroll
                for (int e = 0; e < DPT; ++e) {
                    dv[e] = top - e >= 0 ? (int)hc[top - e] : 0;
                    local += dv[e];
                }
                const int pre = col_exscan<WPC>(local, redi);
                if (want && pre < kk && kk <= pre + local) {
                    int cum = pre;
#pragma unroll
                    for (int e = 0; e < DPT; ++e) {
                        if (cum < kk && kk <= cum + dv[e]) { s_dig[c] = top - e; s_kk[c] = kk - cum; }
                        cum += dv[e];
                    }
                }
                __syncthreads();
                if (want) {
                    prefix |= (uint32_t)s_dig[c] << shift;
                    mask |= 255u << shift;
                    kk = s_kk[c];
                }
                __syncthreads();
            }
            if (want && u == 0) s_val[c][t] = ordered_to_float(prefix);
        }
    }
    __syncthreads();

    if (a.esamples) {
        // discarded mass of each top-k: the elements below x_k, plus the ties
        // at x_k beyond the k-th, in the frame of the row maximum m
        float el[8];
        int ge[8];
        float xk[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) { el[t] = 0.f; ge[t] = 0; xk[t] = t < a.n_k ? s_val[c][t] : INFINITY; }
        for (int j = u; j < n; j += TPC) {
            const float x = xr[j];
            const float e = __builtin_amdgcn_exp2f(x - m);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                if (x < xk[t]) el[t] += e;
                else ++ge[t];
            }
        }
        float ev = NAN;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if (t < a.n_k) {                       // uniform: every thread holds n_k
                const float es = col_sum<WPC>(el[t], redf);
                const int gs = (int)col_sum<WPC>((float)ge[t], redf);
                if (u == t) ev = es + (float)(gs - a.ks[t]) * __builtin_amdgcn_exp2f(xk[t] - m);
            }
        }
        if (live && u < a.n_k)
            a.esamples[(((size_t)s * a.n_k + u) * a.Hq + hh) * a.Lq + ii] = n > a.ks[u] ? ev : NAN;
    }
    if (live && u < a.n_k) {
        const int t = u;
        const float xk = s_val[c][t];
        a.samples[(((size_t)s * a.n_k + t) * a.Hq + hh) * a.Lq + ii] =
            n > a.ks[t] ? (a.pre ? xk * 0.69314718055994531f : exp2f(xk - lse2)) : NAN;
    }
#endif
}

// --------------------------------------------- tiled calibration of prefill rows
// Calibration of whole causal prefills (q_pos0 = 0, Lq = Lk) in the tile
// layout of the prefill kernel: a workgroup of 4 waves takes 32 query rows
// per wave of one KV group and streams the group's K tiles of 64 keys through
// LDS three times (two tile buffers, one tile ahead), recomputing the scores
// on MFMA each time instead of keeping them, so K is read once per 32 * RBW
// rows and two workgroups fit on a CU (one's select phases overlap the
// other's sweeps):
//   sweep A  per row: maximum M, minimum, sum of scores and the softmax sum
//            (the row log-sum-exp lse2);
//   sweep B  a histogram of 256 bins over a window below M: the full range
//            for rows shorter than 3 k_max, else the smaller of the full range
//            and 1.1 (M - mean).  The bin of a score x is read off the bits of
//            one fma, fma(x, -bs, M bs + 2^23 + 1): a float in [2^23, 2^24)
//            whose low bits are (M - x) bs + 1 rounded, so the bin is a
//            monotone (non-increasing) function of x.  Counts are 8-bit, four to a
//            word; everything past the window (and the masked keys) goes to a
//            32-bit sink word after the 64 count words, so a row's counts plus
//            its sink add up to the keys swept unless an 8-bit count wrapped.
//            A prefix over the bins gives, for every target k, the bin holding
//            the k-th largest score and its rank inside that bin;
//   sweep C  every lane appends the elements of its two rows whose fma bits
//            equal a target bin's to a private region of 32 slots, one row
//            from each end (no atomics, no branches).  Then one lane per
//            (row, target) reads the row's four regions and keeps the largest
//            members of the target bin in a register sorting network of up to
//            32 (the smallest when the rank is nearer the bottom of the bin),
//            so the member of that rank is exact whenever it is within 32 of
//            either end of its bin.
// A row whose counts wrapped, whose k-th largest lies past the window, whose
// members do not fit the regions, or whose k-th largest is more than 32 from
// either end of its bin is listed for calib_fixup_kernel, which recomputes it and selects
// exactly by radix select.  Bins are a pure function of the recomputed scores,
// which every sweep forms identically, so the sweeps agree on every element.
constexpr int kCtNB = 256;                      // histogram bins per row (in the window)
constexpr int kCtRowWords = kCtNB / 4 + 1;      // 8-bit counts, + the sink word (also puts rows in other banks)
constexpr uint32_t kCtBinBase = 0x4B000000u;    // bits of 2^23: bin 0
constexpr float kCtBinOffset = 8388609.0f;      // 2^23 + 1
constexpr int kCtSlots = 32;                    // candidate slots per lane (both of its rows)
constexpr int kCtRegion = kCtSlots + 1;         // words between regions: equal slots of the 64 lanes in distinct banks
constexpr int kCtPool = 64 * kCtRegion > 32 * kCtRowWords ? 64 * kCtRegion : 32 * kCtRowWords;   // words per wave
constexpr int kCtNet = 32;                      // registers of the exact-select network
constexpr int kCtMaxK = 4;                      // targets per call on this path
constexpr int kCtEntries = 32 * kCtMaxK;        // (row, target) entries of a wave
static_assert(64 * kCtRegion <= kCtPool && 32 * kCtRowWords <= kCtPool, "histogram and regions in the pool");

constexpr int kCtWaves = 4;
// longest row of the tiled path: the fixup list packs a row into 16 bits, and
// calib_fixup_kernel holds one row of scores in LDS (64 KiB at this length)
constexpr int kCtMaxL = 16384;

template <int D, int G>
struct CtCfg {
    static constexpr int HPW = G < kCtWaves ? G : kCtWaves;   // query heads per workgroup
    static constexpr int RBW = kCtWaves / HPW;      // 32-row blocks per workgroup
    static constexpr int BMT = 32 * RBW;            // query rows per workgroup
    static constexpr int BN = 64;                   // keys per tile
    static constexpr int KSTEPS = D / 32;
    static constexpr int CPR = D / 8;               // 16-byte chunks per K row
    static constexpr int RPI = 64 / CPR;            // K rows per 1 KiB load instruction
    static constexpr int KTILE = BN * D * 2;
    static constexpr int NLD = KTILE / 1024 / kCtWaves;   // load instructions per wave per tile
    static_assert(NLD >= 1, "a tile must give every wave a load");
};

struct CalibTArgs {
    const uint16_t* q; const uint16_t* k;
    int S, Hq, Hkv, L;
    float xscale, scale;
    int ks[kCtMaxK]; int n_k; int kmax;
    float* samples;            // [S][n_k][Hq][L]
    int pre;                   // samples are k-th largest scores (pre-softmax)
    unsigned* fix_count;       // entries listed for the exact fixup
    uint4* fix_list;           // (sequence, head, row | target << 16, lse2 bits)
};

__device__ __forceinline__ void ct_wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }


// LDS accesses written out: the compiler cannot tell an LDS atomic or store
// from the buffer-to-LDS K loads in flight into the other tile buffer and
// would wait for those loads before every one of them.  The histogram and
// the candidate regions are never a target of those loads.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return (uint32_t)(size_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void lds_add(uint32_t addr, uint32_t v) {
    asm volatile("ds_add_u32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_store(uint32_t addr, float v) {
    asm volatile("ds_write_b32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}
// c + hit and c - hit in one VALU instruction each: the lane mask of the hits
// (compares straight into a scalar register pair) is the carry (borrow)
// input of an integer add (subtract) of zero
__device__ __forceinline__ uint64_t eq_mask(uint32_t a, uint32_t b) { return __builtin_amdgcn_uicmp(a, b, 32); }
__device__ __forceinline__ int add_hit(int c, uint64_t m) {
    int r;
    uint64_t co;
    asm("v_addc_co_u32_e64 %0, %1, %2, 0, %3" : "=v"(r), "=s"(co) : "v"(c), "s"(m));
    return r;
}
__device__ __forceinline__ int sub_hit(int c, uint64_t m) {
    int r;
    uint64_t co;
    asm("v_subb_co_u32_e64 %0, %1, %2, 0, %3" : "=v"(r), "=s"(co) : "v"(c), "s"(m));
    return r;
}

// The member of rank rr of the target bin (fma bits tbits) of a row, counted
// from the top (flip = 0) or from the bottom (flip = ~0), from the candidate
// regions of the row's four lanes (g16 + 16 src; row qb = 0 at the start of a
// region, row qb = 1 at its end; c[src] candidates each).  Members enter an
// N-register network as order-preserving keys xor flip, everything else as 0
// (below every key); the network keeps the N largest, rr <= N.  No branch
// per candidate: the lanes of a wave walk their rows' candidates together.
template <int N>
__device__ __forceinline__ float ct_select(const float* pool, const int (&c)[4], int g16, int qb, uint32_t tbits,
                                           float nbs, float cb, uint32_t flip, int rr) {
    uint32_t r[N];
#pragma unroll
    for (int i = 0; i < N; ++i) r[i] = 0u;
#pragma unroll
    for (int src = 0; src < 4; ++src) {
        const float* reg = pool + kCtRegion * (g16 + 16 * src) + (qb == 0 ? 0 : kCtSlots - 1);
        const int step = qb == 0 ? 1 : -1;
        for (int jj = 0; jj < c[src]; ++jj) {
            const float y = reg[step * jj];
            uint32_t v = __float_as_uint(fmaf(y, nbs, cb)) == tbits ? float_to_ordered(y) ^ flip : 0u;
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const uint32_t hi = max(r[i], v);
                v = min(r[i], v);
                r[i] = hi;
            }
        }
    }
    uint32_t k = r[0];
#pragma unroll
    for (int i = 1; i < N; ++i) k = i == rr - 1 ? r[i] : k;
    return ordered_to_float(k ^ flip);
}

template <int D, int G>
__global__ __launch_bounds__(kCtWaves * 64, 2) void calib_tiled_kernel(CalibTArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
    using C = CtCfg<D, G>;
    constexpr int W = kCtWaves;
    // two K tile buffers as separate objects, so that reads of one are not
    // taken to alias the loads in flight into the other
    __shared__ __attribute__((aligned(16))) unsigned char s_k0[C::KTILE];
    __shared__ __attribute__((aligned(16))) unsigned char s_k1[C::KTILE];
    __shared__ uint32_t s_hist[W][kCtPool];          // per wave: histogram, then the candidate regions
    __shared__ int s_ccnt[W][64][2];                 // candidates per lane and row
    __shared__ int s_lovf[W][16];                    // a lane of the group l16 overran its region
    __shared__ float s_rnbs[W][32], s_rcb[W][32], s_rlse[W][32]; // bin fma operands and lse2 of each row
    __shared__ int s_etb[W][kCtEntries];             // target bin (-1: none, or listed for the fixup)
    __shared__ int s_ecnt[W][kCtEntries];            // members of the target bin
    __shared__ int s_erank[W][kCtEntries];           // rank inside the bin; -1: listed for the fixup
    __shared__ float s_eval[W][kCtEntries];          // the k-th largest score

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, lq = lane >> 4;
    const float NEG_INF = -INFINITY;
    const int n_k = a.n_k;

    // Workgroup w goes to XCD w % 8.  The logical workgroups of one (sequence,
    // head block), which read the same K, are numbered consecutively and dealt
    // to one XCD in order, so that XCD's L2 serves K to all of them (and to
    // all three sweeps); a remainder of fewer than 8 keeps its own order.
    const int nqt = (a.L + C::BMT - 1) / C::BMT;
    const unsigned nhb = (unsigned)(a.Hkv * (G / C::HPW));
    const unsigned nwg = gridDim.x, nfull = nwg & ~7u;
    unsigned w = blockIdx.x;
    if (w < nfull) w = (w & 7u) * (nfull >> 3) + (w >> 3);
    const int qt = nqt - 1 - (int)(w % (unsigned)nqt);        // longest query tiles first
    const unsigned grp = w / (unsigned)nqt;
    const int hb = (int)(grp % nhb);
    const int sq = (int)(grp / nhb);
    const int kv = hb / (G / C::HPW);
    const int hblk = hb % (G / C::HPW);
    const int h = kv * G + hblk * C::HPW + wave % C::HPW;
    const int row0 = qt * C::BMT + (wave / C::HPW) * 32;
    const int wg_row_end = min(a.L, (qt + 1) * C::BMT);
    const int ntiles = (wg_row_end + C::BN - 1) / C::BN;

    const uint16_t* kg = a.k + ((size_t)sq * a.Hkv + kv) * (size_t)a.L * D;
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kg), 0, a.L * D * 2, 0x00020000);

    // Q^T fragments (B operand): query row row0 + 16 qb + l16, dims 32 s + 8 lq + e
    bf16x8 qf[2][C::KSTEPS];
    {
        const uint16_t* qg = a.q + ((size_t)sq * a.Hq + h) * (size_t)a.L * D;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int r = min(row0 + 16 * qb + l16, a.L - 1);
#pragma unroll
            for (int st = 0; st < C::KSTEPS; ++st)
                qf[qb][st] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qg + (size_t)r * D + 32 * st + 8 * lq));
        }
    }
    // K tile staging (XOR-swizzled 16-byte chunks, as in the prefill kernel)
    constexpr int NVO = C::CPR / C::RPI > 0 ? C::CPR / C::RPI : 1;
    int vo[NVO];
#pragma unroll
    for (int j = 0; j < NVO; ++j) {
        const int row = j * C::RPI + lane / C::CPR;
        vo[j] = (lane / C::CPR) * (D * 2) + (((lane % C::CPR) ^ (row % C::CPR)) * 16);
    }
    auto issue_k = [&](unsigned char* dst, int tile) {
#pragma unroll
        for (int i = 0; i < C::NLD; ++i) {
            const int li = wave * C::NLD + i;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                krs, (__attribute__((address_space(3))) void*)(dst + li * 1024), 16,
                vo[li % NVO], (tile * C::BN + li * C::RPI) * (D * 2), 0, 0);
        }
    };
    // K fragments of a tile (A operand): key 16 kb + l16, dims 32 st2 + 8 lq .. + 7
    typedef bf16x8 KFrag[4][C::KSTEPS];
    auto load_k = [&](const unsigned char* buf, KFrag& kf) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int key = 16 * kb + l16;
            const unsigned char* srow = buf + ((key / C::RPI) * 64 + (key % C::RPI) * C::CPR) * 16;
            const int swz = key % C::CPR;
#pragma unroll
            for (int st2 = 0; st2 < C::KSTEPS; ++st2)
                kf[kb][st2] = __builtin_bit_cast(bf16x8, *(const u32x4*)(srow + ((4 * st2 + lq) ^ swz) * 16));
        }
    };
    // raw scores q.k of a tile: keys 16 kb + 4 lq + r of the tile, rows row0 + 16 qb + l16
    auto mfma_k = [&](const KFrag& kf, f32x4 (&st)[2][4]) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st2 = 0; st2 < C::KSTEPS; ++st2) {
                acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb][st2], qf[0][st2], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb][st2], qf[1][st2], acc1, 0, 0, 0);
            }
            st[0][kb] = acc0;
            st[1][kb] = acc1;
        }
    };
    // keys past a row, and rows past L, become -inf (tile j crosses the wave's diagonal)
    auto mask = [&](int j, f32x4 (&st)[2][4]) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int row = row0 + 16 * qb + l16;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (j * C::BN + 16 * kb + 4 * lq + r > row || row >= a.L) st[qb][kb][r] = NEG_INF;
        }
    };
    // Tile tdiag holds keys row0 .. row0 + 31 (the wave's diagonal); tiles
    // before it need no mask, tiles after it are all masked and are skipped.
    const int tdiag = min(row0 / C::BN, ntiles);
    // One pass over the key tiles, software-pipelined: at step j the MFMAs of
    // tile j + 1 run between the VALU work of tile j (`plain`, one basic
    // block), while tile j + 2 loads into the buffer tile j came from.  The
    // diagonal tile is masked and goes to `diag`.  Tile t lives in buffer t & 1;
    // the two buffers are separate objects so that reads of one are not taken
    // to alias the loads in flight into the other.
    auto sweep = [&](auto&& plain, auto&& diag) {
        issue_k(s_k0, 0);
        if (ntiles > 1) {
            issue_k(s_k1, 1);
            __builtin_amdgcn_s_waitcnt(0x0F70 | C::NLD);    // vmcnt(NLD): tile 0 landed, tile 1 may not have
        } else {
            ct_wait_vmem();
        }
        __syncthreads();
        f32x4 sa[2][4], sb[2][4];
        {
            KFrag kf;
            load_k(s_k0, kf);
            mfma_k(kf, sa);
        }
        auto step = [&](int j, unsigned char* load_into, const unsigned char* next_buf, f32x4 (&cur)[2][4],
                        f32x4 (&nxt)[2][4]) {
            ct_wait_vmem();
            __syncthreads();                             // tile j + 1 landed; every wave is done with tile j's buffer
            if (j + 2 < ntiles) issue_k(load_into, j + 2);
            if (j < tdiag) {
                if (j + 1 < ntiles) {
                    KFrag kf;
                    load_k(next_buf, kf);
                    mfma_k(kf, nxt);
                    plain(cur);
                } else {
                    plain(cur);
                }
            } else if (j == tdiag) {
                mask(j, cur);
                diag(cur);
            }
        };
        for (int j = 0; j < ntiles; j += 2) {
            step(j, s_k0, s_k1, sa, sb);
            if (j + 1 < ntiles) step(j + 1, s_k1, s_k0, sb, sa);
        }
        __syncthreads();                                 // both buffers free for the next sweep
    };

    // ======================= sweep A: row statistics ==========================
    float m_l[2] = {NEG_INF, NEG_INF}, l_l[2] = {0.f, 0.f}, mn_l[2] = {INFINITY, INFINITY}, sx_l[2] = {0.f, 0.f};
    // online softmax sum in the frame of the running maximum, branch-free: a
    // row with no key yet keeps m = -inf and l = 0
    auto fold_exp = [&](int qb, float tmax, const f32x4 (&st)[2][4]) {
        const float mnew = fmaxf(m_l[qb], tmax);
        const float mref = mnew == NEG_INF ? 0.f : mnew;
        const float nmc = -mref * a.xscale;
        float sum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) sum += __builtin_amdgcn_exp2f(fmaf(st[qb][kb][r], a.xscale, nmc));
        l_l[qb] = l_l[qb] * __builtin_amdgcn_exp2f((m_l[qb] - mref) * a.xscale) + sum;
        m_l[qb] = mnew;
    };
    sweep(
        [&](f32x4 (&st)[2][4]) {                         // no masked key
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                float tmax = NEG_INF, tmin = INFINITY, tsum = 0.f;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float x = st[qb][kb][r];
                        tmax = fmaxf(tmax, x);
                        tmin = fminf(tmin, x);
                        tsum += x;
                    }
                mn_l[qb] = fminf(mn_l[qb], tmin);
                sx_l[qb] += tsum;
                fold_exp(qb, tmax, st);
            }
        },
        [&](f32x4 (&st)[2][4]) {                         // masked keys: left out of the minimum and sum
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                float tmax = NEG_INF, tmin = INFINITY, tsum = 0.f;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float x = st[qb][kb][r];
                        tmax = fmaxf(tmax, x);
                        const bool ok = x > NEG_INF;
                        tmin = fminf(tmin, ok ? x : INFINITY);
                        tsum += ok ? x : 0.f;
                    }
                mn_l[qb] = fminf(mn_l[qb], tmin);
                sx_l[qb] += tsum;
                fold_exp(qb, tmax, st);
            }
        });
    // the four lanes of a row (16 apart) combine; every one of them gets the result
    float nbs[2], cb[2], lse2[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        float M = fmaxf(m_l[qb], __shfl_xor(m_l[qb], 16));
        M = fmaxf(M, __shfl_xor(M, 32));
        float part = (m_l[qb] == NEG_INF) ? 0.f : l_l[qb] * __builtin_amdgcn_exp2f((m_l[qb] - M) * a.xscale);
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        float mn = fminf(mn_l[qb], __shfl_xor(mn_l[qb], 16));
        mn = fminf(mn, __shfl_xor(mn, 32));
        float sx = sx_l[qb] + __shfl_xor(sx_l[qb], 16);
        sx += __shfl_xor(sx, 32);
        const int n = row0 + 16 * qb + l16 + 1;
        lse2[qb] = M * a.xscale + __log2f(part);
        float w = M - mn;
        if (n >= 3 * a.kmax) w = fminf(w, 1.1f * (M - sx / (float)n));
        w = fmaxf(w, 1e-30f);
        // bins of width w / 253 from M down; |M| bs stays below 2^21, so M bs
        // + 2^23 + 1 rounds by at most 1/2 and the bits of the fma are at
        // least those of 2^23 for every x <= M (coarser bins where the whole
        // row lies within 1.2e-4 relative of M)
        float bs = (float)(kCtNB - 3) / w;
        if (fabsf(M) * bs > 2097152.f) bs = 2097152.f / fabsf(M);
        nbs[qb] = -bs;
        cb[qb] = fmaf(M, bs, kCtBinOffset);
        if (lq == 0) {
            s_rnbs[wave][16 * qb + l16] = nbs[qb];
            s_rcb[wave][16 * qb + l16] = cb[qb];
            s_rlse[wave][16 * qb + l16] = lse2[qb];
        }
    }

    // ======================= sweep B: histograms ==============================
    // fma bits of x, capped at bin 256 (the sink word): word (bin >> 2) gets
    // 1 << 8 (bin & 3); the sink's increment is 1
    uint32_t* hw = s_hist[wave];
    const uint32_t hw_off = lds_offset(hw);
    for (int i = lane; i < kCtPool; i += 64) hw[i] = 0u;    // the sweep's first barrier orders this
    auto hist = [&](f32x4 (&st)[2][4]) {                 // masked keys land in the sink
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const uint32_t rbase = hw_off + (uint32_t)((16 * qb + l16) * kCtRowWords) * 4u;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t bits = min(__float_as_uint(fmaf(st[qb][kb][r], nbs[qb], cb[qb])), kCtBinBase + 256u);
                    lds_add(rbase + (bits & 0x1FCu), 1u << ((bits << 3) & 31u));
                }
        }
    };
    sweep(hist, hist);
    __builtin_amdgcn_s_waitcnt(0xC07F);                 // lgkmcnt(0): the written-out atomics are done
    // every entry starts as "no target"; the lanes that find a target set it after the barrier
    for (int e = lane; e < kCtEntries; e += 64) {
        s_etb[wave][e] = -1;
        s_erank[wave][e] = 0;
        s_eval[wave][e] = __uint_as_float(0x7FC00000u);   // NaN until the exact value is found
    }
    __syncthreads();

    // ---- bin and rank of each target: lane (rl, half) scans 128 bins of row rl
    {
        const int rl = lane & 31, half = lane >> 5;
        const int n = row0 + rl + 1;
        const bool live = row0 + rl < a.L;
        const float lrow = s_rlse[wave][rl];
        uint32_t wv[32];
        int ws[32];                                     // count of each word's four bins
        int local = 0;
#pragma unroll
        for (int w = 0; w < 32; ++w) {
            wv[w] = hw[rl * kCtRowWords + 32 * half + w];
            ws[w] = (int)__builtin_amdgcn_sad_u8(wv[w], 0u, 0u);
            local += ws[w];
        }
        const int other = __shfl_xor(local, 32);
        const int base = half ? other : 0;
        const int sink = (int)hw[rl * kCtRowWords + kCtNB / 4];
        // the sweeps stop after the diagonal tile: every row saw (tdiag + 1) 64 keys
        const bool ovf = local + other + sink != min(tdiag + 1, ntiles) * C::BN;   // an 8-bit count wrapped
        for (int t = 0; t < n_k; ++t) {
            const int kk = a.ks[t];
            const int e = rl * n_k + t;
            if (!(live && n > kk)) continue;
            if (ovf || kk > local + other) {            // wrapped, or the k-th largest lies past the window
                if (half == 0) {
                    s_erank[wave][e] = -1;
                    const unsigned idx = atomicAdd(a.fix_count, 1u);
                    a.fix_list[idx] = make_uint4((unsigned)sq, (unsigned)h, (unsigned)(row0 + rl) | ((unsigned)t << 16),
                                                 __float_as_uint(lrow));
                }
                continue;
            }
            if (base < kk && kk <= base + local) {
                // the word holding the k-th largest, then the bin inside it
                int cum = base, wsel = 0, cbefore = base;
#pragma unroll
                for (int w = 0; w < 32; ++w) {
                    if (cum < kk && kk <= cum + ws[w]) { wsel = w; cbefore = cum; }
                    cum += ws[w];
                }
                uint32_t word = 0u;
#pragma unroll
                for (int w = 0; w < 32; ++w) word = w == wsel ? wv[w] : word;
                cum = cbefore;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int bin = 128 * half + 4 * wsel + i;
                    const int c = (int)((word >> (8 * i)) & 0xffu);
                    if (cum < kk && kk <= cum + c) {
                        s_etb[wave][e] = bin;
                        s_erank[wave][e] = kk - cum;
                        s_ecnt[wave][e] = c;
                    }
                    cum += c;
                }
            }
        }
    }
    __syncthreads();

    // ======================= sweep C: members of the target bins ==============
    // fma bits of each target bin (0: no target; no score's bits are 0)
    uint32_t tb[2][kCtMaxK];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int t = 0; t < kCtMaxK; ++t) {
            const int b = t < n_k ? s_etb[wave][(16 * qb + l16) * n_k + t] : -1;
            tb[qb][t] = b >= 0 ? kCtBinBase + (uint32_t)b : 0u;
        }
    // this lane's region: words 33 lane .. 33 lane + 31; row qb = 0 fills slots
    // 0, 1, .. and row qb = 1 slots 31, 30, ..; each row's next free slot takes
    // the stores of non-members (a later member overwrites it).  Masked keys
    // have the bits of +inf and match no target.
    const uint32_t reg_off = hw_off + (uint32_t)(kCtRegion * lane) * 4u;
    // members so far: row qb = 0 counts up from 0, row qb = 1 down from the
    // last slot (both unclamped; the store slot is clamped to the region)
    int c_up = 0, c_dn = kCtSlots - 1;
    // NT compares per element: one sweep per target count (uniform branch)
    auto collect_sweep = [&](auto nt_tag) {
        constexpr int NT = decltype(nt_tag)::value;
        auto collect = [&](f32x4 (&st)[2][4]) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float x = st[qb][kb][r];
                        const uint32_t bits = __float_as_uint(fmaf(x, nbs[qb], cb[qb]));
                        // bitwise, not short-circuit: no branch per element
                        uint64_t hit = eq_mask(bits, tb[qb][0]);
#pragma unroll
                        for (int t = 1; t < NT; ++t) hit |= eq_mask(bits, tb[qb][t]);
                        if (qb == 0) {
                            lds_store(reg_off + (uint32_t)min(c_up, kCtSlots - 1) * 4u, x);
                            c_up = add_hit(c_up, hit);
                        } else {
                            lds_store(reg_off + (uint32_t)max(c_dn, 0) * 4u, x);
                            c_dn = sub_hit(c_dn, hit);
                        }
                    }
            }
        };
        sweep(collect, collect);
    };
    switch (n_k) {
        case 1: collect_sweep(std::integral_constant<int, 1>{}); break;
        case 2: collect_sweep(std::integral_constant<int, 2>{}); break;
        case 3: collect_sweep(std::integral_constant<int, 3>{}); break;
        default: collect_sweep(std::integral_constant<int, kCtMaxK>{}); break;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);                 // lgkmcnt(0): the written-out stores are done
    const int cc[2] = {c_up, kCtSlots - 1 - c_dn};
    s_ccnt[wave][lane][0] = cc[0];
    s_ccnt[wave][lane][1] = cc[1];
    {
        // the two rows' members and their scratch slots must not meet
        int o = cc[0] + cc[1] > kCtSlots - 1 ? 1 : 0;
        o |= __shfl_xor(o, 16);
        o |= __shfl_xor(o, 32);
        if (lq == 0) s_lovf[wave][l16] = o;
    }
    __syncthreads();

    // ---- exact value: one lane per (row, target) entry, 64 entries at a time
    {
        const float* pool = reinterpret_cast<const float*>(hw);
        for (int e0 = 0; e0 < 32 * n_k; e0 += 64) {
            const int e = e0 + lane;
            const bool valid = e < 32 * n_k;
            const int rl = valid ? e / n_k : 0;
            const int qb = rl >> 4, g16 = rl & 15;
            const int tbe = valid ? s_etb[wave][e] : -1;
            const int rank = valid ? s_erank[wave][e] : 0;
            const int m = valid ? s_ecnt[wave][e] : 0;
            bool act = tbe >= 0 && rank > 0;
            // the rank counted from the nearer end of the bin
            const bool top = rank <= m - rank + 1;
            const int rr = top ? rank : m - rank + 1;
            if (act && (s_lovf[wave][g16] || rr > kCtNet)) {
                s_erank[wave][e] = -1;
                const unsigned idx = atomicAdd(a.fix_count, 1u);
                const int t = e - rl * n_k;
                a.fix_list[idx] = make_uint4((unsigned)sq, (unsigned)h, (unsigned)(row0 + rl) | ((unsigned)t << 16),
                                             __float_as_uint(s_rlse[wave][rl]));
                act = false;
            }
            // the network needs rr registers: the smallest of 4, 8, 16, 32 that
            // covers every lane of the wave (all lanes take part: uniform)
            int need = act ? rr : 0;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) need = max(need, __shfl_xor(need, o));
            if (need == 0) continue;
            int c[4];
#pragma unroll
            for (int src = 0; src < 4; ++src) c[src] = act ? s_ccnt[wave][g16 + 16 * src][qb] : 0;   // <= 31: no overrun
            const float rnbs = s_rnbs[wave][rl], rcb = s_rcb[wave][rl];
            const uint32_t tbits = act ? kCtBinBase + (uint32_t)tbe : 0u;
            const uint32_t flip = top ? 0u : ~0u;
            float val;
            if (need <= 4) val = ct_select<4>(pool, c, g16, qb, tbits, rnbs, rcb, flip, rr);
            else if (need <= 8) val = ct_select<8>(pool, c, g16, qb, tbits, rnbs, rcb, flip, rr);
            else if (need <= 16) val = ct_select<16>(pool, c, g16, qb, tbits, rnbs, rcb, flip, rr);
            else val = ct_select<32>(pool, c, g16, qb, tbits, rnbs, rcb, flip, rr);
            if (act) s_eval[wave][e] = val;
        }
    }
    __syncthreads();

    // ---- samples: lanes 0..15 hold rows l16 and 16 + l16
    if (lq == 0) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int row = row0 + 16 * qb + l16;
            if (row >= a.L) continue;
            for (int t = 0; t < n_k; ++t) {
                const int e = (16 * qb + l16) * n_k + t;
                const size_t o = (((size_t)sq * n_k + t) * a.Hq + h) * a.L + row;
                if (row + 1 <= a.ks[t]) { a.samples[o] = NAN; continue; }
                if (s_erank[wave][e] < 0) continue;     // the fixup writes it
                const float xk = s_eval[wave][e];
                a.samples[o] = a.pre ? xk * a.scale : exp2f(fmaf(xk, a.xscale, -lse2[qb]));
            }
        }
    }
#endif
}

// Exact samples of the listed (sequence, head, row, target) entries: the row's
// scores from plain dot products into LDS, then a radix select (8-bit digits
// of the order-preserving key, from the top) of the k-th largest.  Grid-stride
// over the entries the tiled kernel listed.
template <int D>
__global__ __launch_bounds__(256) void calib_fixup_kernel(CalibTArgs a) {
    extern __shared__ float fx[];                            // scores of one row
    __shared__ uint32_t s_h[256];
    __shared__ int s_dig, s_rem;
    constexpr int LPR = D / 8;                               // lanes per key row (8 bf16 per lane)
    constexpr int RPW = 64 / LPR;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sub = lane % LPR, grp = lane / LPR;
    const unsigned total = *a.fix_count;
    for (unsigned e = blockIdx.x; e < total; e += gridDim.x) {
        const uint4 ent = a.fix_list[e];
        const int sq = (int)ent.x, h = (int)ent.y, row = (int)(ent.z & 0xffffu), t = (int)(ent.z >> 16);
        const float lse2 = __uint_as_float(ent.w);
        const int n = row + 1;
        const int g = a.Hq / a.Hkv;
        const uint16_t* qr = a.q + (((size_t)sq * a.Hq + h) * a.L + row) * D;
        const uint16_t* kg = a.k + ((size_t)sq * a.Hkv + h / g) * (size_t)a.L * D;
        float qv[8];
        {
            const u32x4 u = *(const u32x4*)(qr + 8 * sub);
#pragma unroll
            for (int i = 0; i < 4; ++i) { qv[2 * i] = __uint_as_float(u[i] << 16); qv[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u); }
        }
        // UN key steps per trip, their loads issued together (keys past the
        // row read its last key and are not stored)
        constexpr int UN = 8;
        for (int j0 = wave * RPW; j0 < n; j0 += 4 * RPW * UN) {
            u32x4 u[UN];
#pragma unroll
            for (int s2 = 0; s2 < UN; ++s2)
                u[s2] = *(const u32x4*)(kg + (size_t)min(j0 + s2 * 4 * RPW + grp, n - 1) * D + 8 * sub);
#pragma unroll
            for (int s2 = 0; s2 < UN; ++s2) {
                const int j = j0 + s2 * 4 * RPW + grp;
                float dot = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    dot = fmaf(qv[2 * i], __uint_as_float(u[s2][i] << 16), dot);
                    dot = fmaf(qv[2 * i + 1], __uint_as_float(u[s2][i] & 0xffff0000u), dot);
                }
#pragma unroll
                for (int o = 1; o < LPR; o <<= 1) dot += __shfl_xor(dot, o);
                if (j < n && sub == 0) fx[j] = dot;
            }
        }
        __syncthreads();
        uint32_t prefix = 0u, mask = 0u;
        int rem = a.ks[t];
        for (int shift = 24; shift >= 0; shift -= 8) {
            s_h[tid] = 0u;
            __syncthreads();
            for (int j = tid; j < n; j += 256) {
                const uint32_t key = float_to_ordered(fx[j]);
                if ((key & mask) == prefix) atomicAdd(&s_h[(key >> shift) & 255u], 1u);
            }
            __syncthreads();
            // the digit that holds the rem-th largest, counted from the top:
            // lane l of wave 0 sums bins 255 - 4 l .. 252 - 4 l, a prefix over
            // the lanes gives the count above each lane's bins, and the one
            // lane whose range covers rem finds the digit among its four
            if (wave == 0) {
                int c[4], sum = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) { c[i] = (int)s_h[255 - 4 * lane - i]; sum += c[i]; }
                int incl = sum;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int w = __shfl_up(incl, o);
                    if (lane >= o) incl += w;
                }
                int cum = incl - sum;
                if (cum < rem && rem <= incl) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if (cum + c[i] >= rem) { s_dig = 255 - 4 * lane - i; s_rem = rem - cum; break; }
                        cum += c[i];
                    }
                }
            }
            __syncthreads();
            prefix |= (uint32_t)s_dig << shift;
            mask |= 255u << shift;
            rem = s_rem;
            __syncthreads();
        }
        if (tid == 0) {
            const float xk = ordered_to_float(prefix);
            const size_t o = (((size_t)sq * a.n_k + t) * a.Hq + h) * a.L + row;
            a.samples[o] = a.pre ? xk * a.scale : exp2f(fmaf(xk, a.xscale, -lse2));
        }
        __syncthreads();                                     // fx is rewritten by the next entry
    }
}

// ------------------------------------------------------------------ host side
int launch_calib_accumulate(const float* samples, const float* esamples, int S, int n_k, int Hq, int Lq,
                            int q_pos0, double* sum, double* sumsq, int* count, double* esum, int n_rows,
                            hipStream_t s);

// score columns per workgroup: 16 columns of at most 2048 keys, halving the
// columns each time the longest causal row doubles (0: longer than 32768)
static int calib_columns(int keys) {
    int c = 16;
    while (c > 1 && keys > 32768 / c) c >>= 1;
    return keys <= 32768 / c ? c : 0;
}

bool calib_bf16_supported(int d, int S, int Hq, int Lq, int q_pos0) {
    // the grid is one dimension of at most 2^31 - 1 workgroups (at least one row and head each)
    return (d == 64 || d == 128) && calib_columns(q_pos0 + Lq) > 0 &&
           (long long)S * Hq * Lq < (1LL << 31);
}

template <int D, int C>
static int launch_calib_variant(const CalibKArgs& a, hipStream_t s) {
    const size_t smem = (size_t)C * a.nks * sizeof(float) + (size_t)kCalHistWords * sizeof(uint32_t);
    const hipError_t e = hipFuncSetAttribute((const void*)calib_bf16_kernel<D, C>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((calib_bf16_kernel<D, C>), dim3(a.nwg), dim3(kCalThreads), smem, s, a);
    return hipGetLastError();
}

template <int D>
static int launch_calib_d(const CalibKArgs& a, int cols, hipStream_t s) {
    switch (cols) {
        case 16: return launch_calib_variant<D, 16>(a, s);
        case 8: return launch_calib_variant<D, 8>(a, s);
        case 4: return launch_calib_variant<D, 4>(a, s);
        case 2: return launch_calib_variant<D, 2>(a, s);
        default: return launch_calib_variant<D, 1>(a, s);
    }
}

template <int D, int G>
static int launch_tiled_variant(const CalibTArgs& a, hipStream_t s) {
    using C = CtCfg<D, G>;
    const unsigned nwg = (unsigned)((a.L + C::BMT - 1) / C::BMT) * (unsigned)(a.Hkv * (G / C::HPW)) * (unsigned)a.S;
    hipLaunchKernelGGL((calib_tiled_kernel<D, G>), dim3(nwg), dim3(kCtWaves * 64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the listed entries (a few hundred per million): one workgroup each, up
    // to 2048 at once; every workgroup reads the count and exits when there is
    // nothing left for it
    const size_t smem = (size_t)a.L * sizeof(float);
    if (smem > 48 * 1024) {
        e = hipFuncSetAttribute((const void*)calib_fixup_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)smem);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((calib_fixup_kernel<D>), dim3(2048), dim3(256), smem, s, a);
    return hipGetLastError();
}

template <int D>
static int launch_tiled_d(const CalibTArgs& a, int G, hipStream_t s) {
    switch (G) {
        case 1: return launch_tiled_variant<D, 1>(a, s);
        case 2: return launch_tiled_variant<D, 2>(a, s);
        case 4: return launch_tiled_variant<D, 4>(a, s);
        case 8: return launch_tiled_variant<D, 8>(a, s);
        default: return launch_tiled_variant<D, 16>(a, s);
    }
}

// whole causal prefills of up to kCtMaxL keys with at most four targets and no
// discarded-mass samples take the tiled kernel
static bool tiled_path(const CalibParams& p) {
    const int G = p.Hq / p.Hkv;
    // one grid dimension: (query tiles of at most 32 rows) x Hq x S workgroups at most
    return p.q_pos0 == 0 && p.Lq == p.Lk && p.Lk <= kCtMaxL && p.esum == nullptr && p.n_k <= kCtMaxK &&
           (G == 1 || G == 2 || G == 4 || G == 8 || G == 16) && (long long)((p.Lq + 31) / 32) * p.Hq * p.S < (1LL << 31);
}

int launch_calibrate_bf16(const CalibParams& p, float* samples_ws, hipStream_t s) {
    if (tiled_path(p)) {
        CalibTArgs t = {};
        t.q = (const uint16_t*)p.q; t.k = (const uint16_t*)p.k;
        t.S = p.S; t.Hq = p.Hq; t.Hkv = p.Hkv; t.L = p.Lq;
        t.xscale = p.scale * kLog2e; t.scale = p.scale;
        t.kmax = 0;
        for (int i = 0; i < kCtMaxK; ++i) {
            t.ks[i] = i < p.n_k ? p.ks[i] : 0;
            if (i < p.n_k && p.ks[i] > t.kmax) t.kmax = p.ks[i];
        }
        t.n_k = p.n_k;
        t.samples = samples_ws;
        t.pre = p.pre ? 1 : 0;
        // workspace: samples, the fixup count, the fixup list
        const size_t n = (size_t)p.S * p.n_k * p.Hq * p.Lq;
        char* base = (char*)samples_ws + ((n * sizeof(float) + 255) & ~(size_t)255);
        t.fix_count = (unsigned*)base;
        t.fix_list = (uint4*)(base + 256);
        int e = launch_fill_u32(t.fix_count, 4, 0u, s);
        if (e != hipSuccess) return e;
        e = p.d == 64 ? launch_tiled_d<64>(t, p.Hq / p.Hkv, s) : launch_tiled_d<128>(t, p.Hq / p.Hkv, s);
        if (e != hipSuccess) return e;
        return launch_calib_accumulate(samples_ws, nullptr, p.S, p.n_k, p.Hq, p.Lq, p.q_pos0, p.sum, p.sumsq,
                                       p.count, nullptr, p.n_rows, s);
    }
    CalibKArgs a = {};
    a.q = (const uint16_t*)p.q; a.k = (const uint16_t*)p.k;
    a.S = p.S; a.Hq = p.Hq; a.Hkv = p.Hkv; a.Lq = p.Lq; a.Lk = p.Lk; a.q_pos0 = p.q_pos0;
    a.xscale = p.scale * kLog2e;
    for (int t = 0; t < 8; ++t) a.ks[t] = t < p.n_k ? p.ks[t] : 0;
    a.n_k = p.n_k;
    a.samples = samples_ws;
    a.pre = p.pre ? 1 : 0;
    // the discarded-mass samples follow the value samples in the workspace
    a.esamples = p.esum ? samples_ws + (size_t)p.S * p.n_k * p.Hq * p.Lq : nullptr;
    const int keys = p.q_pos0 + p.Lq;
    const int cols = calib_columns(keys);
    // 16-key tiles, plus 4 floats so that consecutive columns start in different LDS banks
    a.nks = (keys + 15) / 16 * 16 + 4;
    const int g = p.Hq / p.Hkv;
    int gh = cols;
    while (g % gh) gh >>= 1;
    a.gh = gh;
    a.rb = cols / gh;
    a.nblk = (p.Lq + a.rb - 1) / a.rb;
    a.ngh = p.Hq / gh;
    a.nwg = (unsigned)a.nblk * (unsigned)a.ngh * (unsigned)p.S;
    const int e = p.d == 64 ? launch_calib_d<64>(a, cols, s) : launch_calib_d<128>(a, cols, s);
    if (e != hipSuccess) return e;
    return launch_calib_accumulate(samples_ws, a.esamples, p.S, p.n_k, p.Hq, p.Lq, p.q_pos0, p.sum, p.sumsq,
                                   p.count, p.esum, p.n_rows, s);
}

}  // namespace topth
