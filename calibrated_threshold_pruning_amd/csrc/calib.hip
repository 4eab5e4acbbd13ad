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

int launch_calibrate_bf16(const CalibParams& p, float* samples_ws, hipStream_t s) {
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
