// Row-per-workgroup kernels: one workgroup owns one attention row end to end
// (scores in LDS, row statistics, threshold, compensation).  They serve the
// float32 element type for every operation and the bfloat16 prefill and
// calibration until the tiled kernels take over those shapes.
//
// Method: "Top-Theta Attention: Sparsifying Transformers by Compensated
// Thresholding" -- Eq. 1-3 (scores, softmax, SV), Sec. 3 (keep s >= theta),
// Sec. 3.1 Algorithm 1 (k-th largest per row, post-softmax), Sec. 3.2.1 Eq. 4
// (exact SDC: kept weights keep the full denominator), Sec. 3.2.2 Eq. 5-7 (VMC).
// With kFlagPre the same kernels run the pre-softmax form: keep a >= theta on
// the scores, calibrate the k-th largest score (Algorithm 1 as printed) and the
// discarded mass of the top-k, and scale the kept softmax values by one of the
// Sec. 3.2.1 estimates of E~ (exact, exp-threshold, offline-calibrated).
#include "topth_internal.h"

#include <math.h>

namespace topth {

enum RowMode { kRowDecode = 0, kRowPrefill = 1, kRowCalib = 2 };

struct RowArgs {
    const void* q; const void* k; const void* v; const int* seq_lens;
    int B, Hq, Hkv, Lq, Lk;       // Lk: key rows per (b, kv) in memory (Lmax for decode)
    float xscale;                 // scale * log2(e): scores are kept in the log2 domain
    int q_pos0;
    const float* theta; int n_rows;
    const float* mu;              // decode: [B][Hkv][d]; prefill: prefix means [B][Hkv][L][d]
    unsigned flags;
    void* out; int* kept_count; float* beta;
    int ks[8]; int n_k; float* samples;   // calibration: [S][n_k][Hq][Lq]
    float* esamples;                      // pre-softmax calibration: discarded mass, same shape, or NULL
    const float* e_tilde; float gamma;    // pre-softmax SDC estimates
    uint32_t* masks; int mask_words;      // decode: kept-key bitmasks [B][Hq][mask_words]
    unsigned char* kept_mask;             // optional byte mask, [rows][Lk]
    // decode GQA selection variants (Sec. 4.6), two passes: 1 writes each
    // head's kept-key bits to masks; 2 reads the group's bits, loads a key
    // when at least min_votes heads keep it and keeps, per head, its own
    // loaded keys or (augment) all of them
    int gqa_pass, min_votes, augment;
};

constexpr int kRowThreads = 256;
constexpr int kRowMaxKeysDecl = 32768;   // longest row the row kernels hold in LDS

__device__ __forceinline__ float block_max(float v, float* red) {
    v = wave_max(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < kRowThreads / 64; ++i) r = fmaxf(r, red[i]);
    return r;
}
__device__ __forceinline__ float block_sum(float v, float* red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float r = 0.f;
    for (int i = 0; i < kRowThreads / 64; ++i) r += red[i];
    return r;
}
__device__ __forceinline__ int block_sum_i(int v, int* red) {
    v = wave_sum_i(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    int r = 0;
    for (int i = 0; i < kRowThreads / 64; ++i) r += red[i];
    return r;
}

// k-th largest (1-based) of xs[0..n) by a most-significant-digit-first radix
// select over order-preserving 32-bit keys, 8 bits per pass.
__device__ float block_kth_largest(const float* xs, int n, int k, unsigned* hist, int* sel) {
    uint32_t prefix = 0, mask = 0;
    int kk = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = threadIdx.x; i < 256; i += kRowThreads) hist[i] = 0;
        __syncthreads();
        for (int j = threadIdx.x; j < n; j += kRowThreads) {
            uint32_t u = float_to_ordered(xs[j]);
            if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            int cum = 0, d = 0;
            for (d = 255; d > 0; --d) {
                int c = (int)hist[d];
                if (cum + c >= kk) break;
                cum += c;
            }
            sel[0] = d;
            sel[1] = kk - cum;
        }
        __syncthreads();
        prefix |= (uint32_t)sel[0] << shift;
        mask |= 255u << shift;
        kk = sel[1];
        __syncthreads();
    }
    return ordered_to_float(prefix);
}

template <typename T, int D, int MODE>
__global__ __launch_bounds__(kRowThreads) void row_kernel(RowArgs a) {
    extern __shared__ float xs[];             // scores (log2 domain), then weights
    __shared__ float qs[D];
    __shared__ float redf[kRowThreads / 64];
    __shared__ int redi[kRowThreads / 64];
    __shared__ unsigned hist[256];
    __shared__ int sel[2];
    __shared__ uint32_t keepbits[MODE == kRowDecode ? kRowMaxKeysDecl / 32 : 1];

    const int row = blockIdx.x;
    const int i = row % a.Lq;
    const int h = (row / a.Lq) % a.Hq;
    const int b = row / (a.Lq * a.Hq);
    const int g = a.Hq / a.Hkv;
    const int kv = h / g;
    int n;
    if (MODE == kRowDecode) n = min(max(a.seq_lens[b], 1), a.Lk);   // clamp to [1, Lmax]
    else if (MODE == kRowPrefill) n = i + 1;
    else n = a.q_pos0 + i + 1;
    const int rowid = n - 1;

    const T* qrow = (const T*)a.q + ((size_t)(b * a.Hq + h) * a.Lq + i) * D;
    for (int t = threadIdx.x; t < D; t += kRowThreads) qs[t] = Elem<T>::load(qrow + t);
    __syncthreads();

    // Eq. 1: scores of the causal row, scaled by 1/sqrt(d) and log2(e)
    const T* kbase = (const T*)a.k + (size_t)(b * a.Hkv + kv) * a.Lk * D;
    float mloc = -INFINITY;
    for (int j = threadIdx.x; j < n; j += kRowThreads) {
        const T* kr = kbase + (size_t)j * D;
        float acc = 0.f;
#pragma unroll 8
        for (int t = 0; t < D; ++t) acc = fmaf(qs[t], Elem<T>::load(kr + t), acc);
        const float x = acc * a.xscale;
        xs[j] = x;
        mloc = fmaxf(mloc, x);
    }
    const float m = block_max(mloc, redf);
    float lloc = 0.f;
    for (int j = threadIdx.x; j < n; j += kRowThreads) lloc += exp2f(xs[j] - m);
    const float lse2 = m + __log2f(block_sum(lloc, redf));   // Eq. 2 denominator, log2 domain

    const bool pre = (a.flags & kFlagPre) != 0;
    if (MODE == kRowCalib) {
        // Algorithm 1: per target k, the k-th largest s of the row (post-softmax)
        // or the k-th largest score a itself (pre-softmax)
        for (int t = 0; t < a.n_k; ++t) {
            const int kk = a.ks[t];
            float val = NAN, ev = NAN;
            if (n > kk) {
                const float xk = block_kth_largest(xs, n, kk, hist, sel);
                val = pre ? xk * 0.69314718055994531f : exp2f(xk - lse2);
                if (a.esamples) {
                    // discarded mass of the top-k in the frame of the row maximum:
                    // the elements below x_k, plus the ties at x_k beyond the k-th
                    float el = 0.f;
                    int ge = 0;
                    for (int j = threadIdx.x; j < n; j += kRowThreads) {
                        const float x = xs[j];
                        if (x < xk) el += exp2f(x - m);
                        else ++ge;
                    }
                    el = block_sum(el, redf);
                    ge = block_sum_i(ge, redi);
                    ev = el + (float)(ge - kk) * exp2f(xk - m);
                }
            }
            if (threadIdx.x == 0) {
                const size_t o = (((size_t)b * a.n_k + t) * a.Hq + h) * a.Lq + i;
                a.samples[o] = val;
                if (a.esamples) a.esamples[o] = ev;
            }
        }
        return;
    }

    // Sec. 3: keep s >= theta  <=>  x >= log2(theta) + lse2 (post-softmax), or
    // a >= theta  <=>  x >= theta * log2(e) (pre-softmax)
    const float th = a.theta[(size_t)h * a.n_rows + min(rowid, a.n_rows - 1)];
    const float T2 = pre ? pre_log2_threshold(th) : log2_threshold(th, lse2);
    if (MODE == kRowDecode) {
        for (int w = threadIdx.x; w < (n + 31) / 32; w += kRowThreads) keepbits[w] = 0u;
        __syncthreads();
    }
    if (MODE == kRowDecode && a.gqa_pass == 1) {
        for (int j = threadIdx.x; j < n; j += kRowThreads)
            if (xs[j] >= T2) atomicOr(&keepbits[j >> 5], 1u << (j & 31));
        __syncthreads();
        uint32_t* mrow = a.masks + (size_t)(b * a.Hq + h) * a.mask_words;
        for (int w = threadIdx.x; w < a.mask_words; w += kRowThreads)
            mrow[w] = (w < (n + 31) / 32) ? keepbits[w] : 0u;
        return;
    }
    int cnt = 0;
    float mass = 0.f;
    for (int j = threadIdx.x; j < n; j += kRowThreads) {
        const float x = xs[j];
        bool keep = x >= T2;
        if (MODE == kRowDecode && a.gqa_pass == 2) {
            int votes = 0;
            for (int hh = 0; hh < g; ++hh)
                votes += (a.masks[(size_t)(b * a.Hq + kv * g + hh) * a.mask_words + (j >> 5)] >> (j & 31)) & 1u;
            keep = votes >= a.min_votes && (a.augment || keep);
        }
        const float w = keep ? exp2f(x - lse2) : 0.f;   // exact SDC: weight = s
        xs[j] = w;
        cnt += keep;
        mass += w;
        if (MODE == kRowDecode && keep) atomicOr(&keepbits[j >> 5], 1u << (j & 31));
        if (a.kept_mask) a.kept_mask[(size_t)row * a.Lk + j] = keep ? 1 : 0;
    }
    if (MODE == kRowPrefill && a.kept_mask)
        for (int j = n + threadIdx.x; j < a.Lk; j += kRowThreads) a.kept_mask[(size_t)row * a.Lk + j] = 0;
    cnt = block_sum_i(cnt, redi);
    mass = block_sum(mass, redf);
    __syncthreads();

    const bool renorm = (a.flags & 2u) != 0;
    const bool vmc = (a.flags & 1u) != 0;
    // Eq. 4 scale of the kept softmax values and Eq. 6 beta; the estimates of
    // E~ relative to the full denominator e^lse: exp-threshold gamma (n - k~)
    // e^(theta - lse), offline E~ e^(max - lse) (E~ is relative to the row max)
    float etn = 0.f;
    if (a.flags & kFlagExpth) etn = a.gamma * (float)(n - cnt) * exp2f(th * kLog2e - lse2);
    if (a.flags & kFlagOffline) etn = a.e_tilde[(size_t)h * a.n_rows + min(rowid, a.n_rows - 1)] * exp2f(m - lse2);
    float fsc, beta;
    sdc_scale(a.flags, mass, cnt, etn, fsc, beta);
    const T* vbase = (const T*)a.v + (size_t)(b * a.Hkv + kv) * a.Lk * D;
    T* orow = (T*)a.out + ((size_t)(b * a.Hq + h) * a.Lq + i) * D;
    const float* mu = nullptr;
    if (vmc && !renorm) {
        mu = (MODE == kRowDecode) ? a.mu + (size_t)(b * a.Hkv + kv) * D
                                  : a.mu + ((size_t)(b * a.Hkv + kv) * a.Lq + i) * D;
    }
    for (int t = threadIdx.x; t < D; t += kRowThreads) {
        float acc = 0.f;
        for (int j = 0; j < n; ++j) {
            const float w = xs[j];
            if (w != 0.f) acc = fmaf(w, Elem<T>::load(vbase + (size_t)j * D + t), acc);
        }
        if (renorm) acc = (cnt > 0) ? acc / mass : 0.f;
        else if (a.flags & (kFlagExpth | kFlagOffline)) acc *= fsc;
        if (mu) acc = fmaf(beta, mu[t], acc);                   // Eq. 7
        Elem<T>::store(orow + t, acc);
    }
    if (threadIdx.x == 0) {
        const size_t o = (size_t)(b * a.Hq + h) * a.Lq + i;
        if (a.kept_count) a.kept_count[o] = cnt;
        if (a.beta) a.beta[o] = beta;
    }
    if (MODE == kRowDecode && a.masks && a.gqa_pass == 0) {
        uint32_t* mrow = a.masks + (size_t)(b * a.Hq + h) * a.mask_words;
        for (int w = threadIdx.x; w < a.mask_words; w += kRowThreads)
            mrow[w] = (w < (n + 31) / 32) ? keepbits[w] : 0u;
    }
}

// number of distinct V rows the GQA group reads: popcount of the OR of its
// heads' kept-key masks (Sec. 4.6).  The mask words live in the decode
// workspace; each is set back to the empty-slot pattern once read.
__global__ void union_count_kernel(uint32_t* masks, int Hq, int Hkv, int mask_words,
                                   int* vrows_read) {
    __shared__ int red[4];
    const int bk = blockIdx.x;
    const int b = bk / Hkv, kv = bk % Hkv;
    const int g = Hq / Hkv;
    int c = 0;
    for (int w = threadIdx.x; w < mask_words; w += blockDim.x) {
        uint32_t u = 0;
        for (int hh = 0; hh < g; ++hh) {
            uint32_t* m = masks + ((size_t)b * Hq + kv * g + hh) * mask_words + w;
            u |= *m;
            *m = kWsSlotEmpty;
        }
        c += __popc(u);
    }
    c = wave_sum_i(c);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) vrows_read[bk] = red[0] + red[1] + red[2] + red[3];
}

// number of V rows the GQA group loads under the vote rule (keys kept by at
// least min_votes of its heads); the mask words are set back to the
// empty-slot pattern once read.
__global__ void votes_count_kernel(uint32_t* masks, int Hq, int Hkv, int mask_words, int min_votes,
                                   int* vrows_read) {
    __shared__ int red[4];
    const int bk = blockIdx.x;
    const int b = bk / Hkv, kv = bk % Hkv;
    const int g = Hq / Hkv;
    int c = 0;
    for (int w = threadIdx.x; w < mask_words; w += blockDim.x) {
        for (int bit = 0; bit < 32; ++bit) {
            int v = 0;
            for (int hh = 0; hh < g; ++hh)
                v += (masks[((size_t)b * Hq + kv * g + hh) * mask_words + w] >> bit) & 1u;
            c += v >= min_votes ? 1 : 0;
        }
    }
    __syncthreads();                      // every word of the group is read before any is reset
    for (int w = threadIdx.x; w < mask_words; w += blockDim.x)
        for (int hh = 0; hh < g; ++hh) masks[((size_t)b * Hq + kv * g + hh) * mask_words + w] = kWsSlotEmpty;
    c = wave_sum_i(c);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0 && vrows_read) vrows_read[bk] = red[0] + red[1] + red[2] + red[3];
}

// mean of the first n = seq_lens[b] V rows, Eq. 5 over the cached rows.  One
// workgroup per (b, KV head): each thread reads 16-byte pieces of rows (CPR
// threads cover a row, RS rows per pass) and keeps float64 partial sums for
// its piece, in row order; the RS partial sums of every column are then added
// in a fixed order, so the result does not depend on scheduling.
constexpr int kVmeanThreads = 512;
template <typename T, int D>
__global__ __launch_bounds__(kVmeanThreads) void vmean_kernel(const T* v, const int* seq_lens, int Hkv,
                                                               int Lmax, float* out) {
    constexpr int EPC = 16 / (int)sizeof(T);          // elements per 16-byte piece
    constexpr int CPR = D / EPC;                      // pieces per row
    constexpr int RS = kVmeanThreads / CPR;           // rows per pass
    __shared__ double part[RS][D];
    const int bk = blockIdx.x;
    const int b = bk / Hkv;
    const int n = min(max(seq_lens[b], 1), Lmax);
    const T* base = v + (size_t)bk * Lmax * D;
    const int c = threadIdx.x % CPR, r0 = threadIdx.x / CPR;
    double acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.0;
    // four rows' loads per trip (rows past n re-read row n - 1 and are not added)
    constexpr int UN = 4;
    for (int j0 = r0; j0 < n; j0 += UN * RS) {
        u32x4 raw[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) raw[u] = *(const u32x4*)(base + (size_t)min(j0 + u * RS, n - 1) * D + c * EPC);
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            if (j0 + u * RS < n) {
                const T* x = reinterpret_cast<const T*>(&raw[u]);
#pragma unroll
                for (int e = 0; e < EPC; ++e) acc[e] += (double)Elem<T>::load(x + e);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < EPC; ++e) part[r0][c * EPC + e] = acc[e];
    __syncthreads();
    for (int t = threadIdx.x; t < D; t += kVmeanThreads) {
        double sum = 0.0;
        for (int r = 0; r < RS; ++r) sum += part[r][t];
        out[(size_t)bk * D + t] = (float)(sum / (double)n);
    }
}

// causal prefix means mu_p = mean of V rows 0..p (Eq. 5 read causally), as a
// scan over chunks of rows, all sums in double in row order within a chunk:
//   chunk c holds rows [64 c, 64 c + 64), the last one also the rows past the
//   last multiple of 64 (so every chunk after the first has at least 64 rows);
//   1. every chunk but the last sums its rows; the sum goes to the slot of
//      the next chunk: D doubles over the first float rows of that chunk's
//      own output region, which its writer reads before overwriting;
//   2. one thread per (group, dimension) turns the slots into running sums
//      (the sum of all rows before the chunk);
//   3. every chunk adds its rows to its slot's sum row by row and writes the
//      means.
// One thread per dimension (D = blockDim.x, at most 128); one workgroup per
// (group, chunk), chunk fastest.
constexpr int kPrefixChunk = 64;

__device__ __forceinline__ int prefix_chunks(int L) { return L / kPrefixChunk > 1 ? L / kPrefixChunk : 1; }
__device__ __forceinline__ int prefix_chunk_end(int c, int nch, int L) {
    return c == nch - 1 ? L : (c + 1) * kPrefixChunk;
}
__device__ __forceinline__ double* prefix_slot(float* mu, int g, int c, int L, int D) {
    return reinterpret_cast<double*>(mu + ((size_t)g * L + (size_t)c * kPrefixChunk) * D);
}

template <typename T>
__global__ void prefix_chunk_sum_kernel(const T* v, int L, float* mu) {
    const int nch = prefix_chunks(L);
    const int D = blockDim.x, t = threadIdx.x, c = blockIdx.x % (nch - 1), g = blockIdx.x / (nch - 1);
    const T* base = v + (size_t)g * L * D;
    double acc = 0.0;
    constexpr int UN = 8;                            // eight rows' loads per trip
    const int p1 = prefix_chunk_end(c, nch, L);
    for (int p0 = c * kPrefixChunk; p0 < p1; p0 += UN) {
        float x[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) x[u] = Elem<T>::load(base + (size_t)min(p0 + u, p1 - 1) * D + t);
#pragma unroll
        for (int u = 0; u < UN; ++u)
            if (p0 + u < p1) acc += (double)x[u];
    }
    prefix_slot(mu, g, c + 1, L, D)[t] = acc;
}

__global__ void prefix_chunk_scan_kernel(int L, int D, int groups, float* mu) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= groups * D) return;
    const int g = i / D, t = i % D;
    const int nch = prefix_chunks(L);
    double run = 0.0;
    // eight chunk sums per trip, their loads issued before any store
    constexpr int UN = 8;
    for (int c0 = 1; c0 < nch; c0 += UN) {
        double x[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) x[u] = prefix_slot(mu, g, min(c0 + u, nch - 1), L, D)[t];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            if (c0 + u < nch) {
                run += x[u];
                prefix_slot(mu, g, c0 + u, L, D)[t] = run;
            }
        }
    }
}

template <typename T>
__global__ void prefix_mean_write_kernel(const T* v, int L, float* mu) {
    __shared__ double s_pre[128];
    const int nch = prefix_chunks(L);
    const int D = blockDim.x, t = threadIdx.x, c = blockIdx.x % nch, g = blockIdx.x / nch;
    // the slot goes through LDS, so that every entry has arrived before any
    // row of the chunk (which the slot overlaps) is written
    s_pre[t] = c == 0 ? 0.0 : prefix_slot(mu, g, c, L, D)[t];
    __syncthreads();
    double acc = s_pre[t];
    const T* base = v + (size_t)g * L * D;
    float* o = mu + (size_t)g * L * D;
    // eight rows per trip, their loads issued together
    constexpr int UN = 8;
    const int p1 = prefix_chunk_end(c, nch, L);
    for (int p0 = c * kPrefixChunk; p0 < p1; p0 += UN) {
        float x[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) x[u] = Elem<T>::load(base + (size_t)min(p0 + u, p1 - 1) * D + t);
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            if (p0 + u < p1) {
                acc += (double)x[u];
                o[(size_t)(p0 + u) * D + t] = (float)(acc / (double)(p0 + u + 1));
            }
        }
    }
}

// Accumulate per-sequence calibration samples into (sum, sumsq, count), in
// sequence order, one thread per (k, head, row).
__global__ void calib_accumulate_kernel(const float* samples, const float* esamples, int S, int n_k,
                                        int Hq, int Lq, int q_pos0, double* sum, double* sumsq,
                                        int* count, double* esum, int n_rows) {
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t per = (size_t)n_k * Hq * Lq;
    if (idx >= per) return;
    const int i = (int)(idx % Lq);
    const int h = (int)((idx / Lq) % Hq);
    const int t = (int)(idx / ((size_t)Lq * Hq));
    const int p = q_pos0 + i;
    if (p >= n_rows) return;
    double s1 = 0.0, s2 = 0.0, e1 = 0.0;
    int c = 0;
    // eight sequences per trip, their loads issued together; the sums still
    // run in sequence order
    constexpr int UN = 8;
    for (int s0 = 0; s0 < S; s0 += UN) {
        float x[UN], ex[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const size_t o = (size_t)min(s0 + u, S - 1) * per + idx;
            x[u] = samples[o];
            ex[u] = esamples ? esamples[o] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            if (s0 + u < S && x[u] == x[u]) {
                s1 += (double)x[u]; s2 += (double)x[u] * (double)x[u]; ++c;
                e1 += (double)ex[u];
            }
        }
    }
    if (c) {
        const size_t o = ((size_t)t * Hq + h) * n_rows + p;
        sum[o] += s1; sumsq[o] += s2; count[o] += c;
        if (esum) esum[o] += e1;
    }
}

// theta = mean + alpha * std of the observed rows; -inf for rows with p+1 <= k;
// other unobserved rows copy the nearest observed row (smaller row on a tie).
constexpr int kFinThreads = 256;
__device__ __forceinline__ float theta_of(const double* sum, const double* sumsq, const int* count,
                                          size_t o, float alpha) {
    const double c = (double)count[o];
    const double mean = sum[o] / c;
    double var = sumsq[o] / c - mean * mean;
    if (var < 0.0) var = 0.0;
    return (float)(mean + (double)alpha * sqrt(var));
}

struct KList { int k[8]; };

// With ETILDE the same rules give the offline estimate of the discarded mass:
// its mean for observed rows, 0 where nothing is discarded (p+1 <= k) or no
// row of the head was observed, the nearest observed row elsewhere.
template <bool ETILDE>
__global__ __launch_bounds__(kFinThreads) void finalize_kernel(
        const double* sum, const double* sumsq, const int* count, int Hq, int n_rows,
        KList ks, float alpha, float* theta) {
    const float none = ETILDE ? 0.f : -INFINITY;
    __shared__ int first_obs[kFinThreads], last_obs[kFinThreads];
    const int t = blockIdx.x / Hq, h = blockIdx.x % Hq;
    const int k = ks.k[t];
    const size_t base = ((size_t)t * Hq + h) * n_rows;
    const int seg = (n_rows + kFinThreads - 1) / kFinThreads;
    const int lo = threadIdx.x * seg, hi = min(n_rows, lo + seg);
    int f = -1, l = -1;
    for (int p = lo; p < hi; ++p)
        if (count[base + p] > 0) { if (f < 0) f = p; l = p; }
    first_obs[threadIdx.x] = f;
    last_obs[threadIdx.x] = l;
    __syncthreads();
    int prev = -1, next = -1;
    for (int u = threadIdx.x - 1; u >= 0 && prev < 0; --u) prev = last_obs[u];
    for (int u = threadIdx.x + 1; u < kFinThreads && next < 0; ++u) next = first_obs[u];
    // forward pass: nearest observed row at or before p
    for (int p = lo; p < hi; ++p) {
        if (count[base + p] > 0) prev = p;
        theta[base + p] = (float)prev;          // temporary: row index as float
    }
    // backward pass: choose between previous and next observed rows
    for (int p = hi - 1; p >= lo; --p) {
        if (count[base + p] > 0) next = p;
        const int pv = (int)theta[base + p];
        float out;
        if (p + 1 <= k) out = none;
        else if (count[base + p] > 0) out = theta_of(sum, sumsq, count, base + p, alpha);
        else if (pv < 0 && next < 0) out = none;
        else {
            int src;
            if (pv < 0) src = next;
            else if (next < 0) src = pv;
            else src = (p - pv <= next - p) ? pv : next;
            out = theta_of(sum, sumsq, count, base + src, alpha);
        }
        theta[base + p] = out;
    }
}

__global__ void fill_u32_kernel(uint32_t* p, size_t n_words, uint32_t value) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = value;
}

// a decode workspace as topth_workspace_init leaves it, up to `end_words`:
// the header words zero, the exchange slots after them empty
__global__ void ws_prepare_kernel(uint32_t* p, size_t header_words, size_t end_words) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < end_words;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = i < header_words ? 0u : kWsSlotEmpty;
}

// ------------------------------------------------------------------ launchers
template <typename T, int D, int MODE>
static int launch_rows(const RowArgs& a, int rows, int smem_floats, hipStream_t s) {
    const size_t smem = (size_t)smem_floats * sizeof(float);
    if (smem > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)row_kernel<T, D, MODE>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((row_kernel<T, D, MODE>), dim3(rows), dim3(kRowThreads), smem, s, a);
    return hipGetLastError();
}

template <int MODE>
static int dispatch_rows(const RowArgs& a, int d, int dtype, int rows, int smem_floats,
                         hipStream_t s) {
    if (dtype == 0) {
        if (d == 64) return launch_rows<float, 64, MODE>(a, rows, smem_floats, s);
        return launch_rows<float, 128, MODE>(a, rows, smem_floats, s);
    }
    if (d == 64) return launch_rows<uint16_t, 64, MODE>(a, rows, smem_floats, s);
    return launch_rows<uint16_t, 128, MODE>(a, rows, smem_floats, s);
}

int rowwise_max_keys() { return kRowMaxKeysDecl; }

size_t decode_rowwise_ws_bytes(int B, int Hq, int Lmax) {
    return (size_t)B * Hq * ((Lmax + 31) / 32) * sizeof(uint32_t);
}

int launch_decode_rowwise(const DecodeParams& p, uint32_t* masks_ws, hipStream_t s) {
    RowArgs a = {};
    a.q = p.q; a.k = p.k; a.v = p.v; a.seq_lens = p.seq_lens;
    a.B = p.B; a.Hq = p.Hq; a.Hkv = p.Hkv; a.Lq = 1; a.Lk = p.Lmax;
    a.xscale = p.scale * kLog2e;
    a.theta = p.theta; a.n_rows = p.n_rows; a.mu = p.v_mean; a.flags = p.flags;
    a.e_tilde = p.e_tilde; a.gamma = p.gamma;
    a.out = p.out; a.kept_count = p.kept_count; a.beta = p.beta; a.kept_mask = p.kept_mask;
    a.mask_words = (p.Lmax + 31) / 32;
    if (p.min_votes > 1 || p.augment) {
        // GQA selection variants: every head's kept bits first, then the outputs
        a.masks = masks_ws;
        a.min_votes = p.min_votes < 1 ? 1 : p.min_votes;
        a.augment = p.augment;
        a.gqa_pass = 1;
        int e = dispatch_rows<kRowDecode>(a, p.d, p.dtype, p.B * p.Hq, p.Lmax, s);
        if (e != hipSuccess) return e;
        a.gqa_pass = 2;
        e = dispatch_rows<kRowDecode>(a, p.d, p.dtype, p.B * p.Hq, p.Lmax, s);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(votes_count_kernel, dim3(p.B * p.Hkv), dim3(256), 0, s,
                           masks_ws, p.Hq, p.Hkv, a.mask_words, a.min_votes, p.vrows_read);
        return hipGetLastError();
    }
    a.masks = p.vrows_read ? masks_ws : nullptr;
    int e = dispatch_rows<kRowDecode>(a, p.d, p.dtype, p.B * p.Hq, p.Lmax, s);
    if (e != hipSuccess) return e;
    if (p.vrows_read) {
        hipLaunchKernelGGL(union_count_kernel, dim3(p.B * p.Hkv), dim3(256), 0, s,
                           masks_ws, p.Hq, p.Hkv, a.mask_words, p.vrows_read);
        e = hipGetLastError();
    }
    return e;
}

template <typename T>
static int launch_prefix_mean_t(const T* v, int groups, int L, int d, float* mu, hipStream_t s) {
    const int nch = L / kPrefixChunk > 1 ? L / kPrefixChunk : 1;
    if (nch > 1) {
        hipLaunchKernelGGL(prefix_chunk_sum_kernel<T>, dim3((unsigned)((nch - 1) * groups)), dim3(d), 0, s, v, L, mu);
        const int n = groups * d;
        hipLaunchKernelGGL(prefix_chunk_scan_kernel, dim3((n + 255) / 256), dim3(256), 0, s, L, d, groups, mu);
    }
    hipLaunchKernelGGL(prefix_mean_write_kernel<T>, dim3((unsigned)(nch * groups)), dim3(d), 0, s, v, L, mu);
    return hipGetLastError();
}

int launch_prefix_mean(const void* v, int groups, int L, int d, int dtype, float* mu, hipStream_t s) {
    if (dtype == 0) return launch_prefix_mean_t((const float*)v, groups, L, d, mu, s);
    return launch_prefix_mean_t((const uint16_t*)v, groups, L, d, mu, s);
}

int launch_prefill_rowwise(const PrefillParams& p, float* mu_ws, hipStream_t s) {
    const bool vmc = (p.flags & 1u) && !(p.flags & 2u);
    if (vmc) {
        const int e = launch_prefix_mean(p.v, p.B * p.Hkv, p.L, p.d, p.dtype, mu_ws, s);
        if (e != hipSuccess) return e;
    }
    RowArgs a = {};
    a.q = p.q; a.k = p.k; a.v = p.v;
    a.B = p.B; a.Hq = p.Hq; a.Hkv = p.Hkv; a.Lq = p.L; a.Lk = p.L;
    a.xscale = p.scale * kLog2e;
    a.theta = p.theta; a.n_rows = p.n_rows; a.mu = mu_ws; a.flags = p.flags;
    a.e_tilde = p.e_tilde; a.gamma = p.gamma;
    a.out = p.out; a.kept_count = p.kept_count; a.beta = p.beta; a.kept_mask = p.kept_mask;
    return dispatch_rows<kRowPrefill>(a, p.d, p.dtype, p.B * p.Hq * p.L, p.L, s);
}

int launch_calib_accumulate(const float* samples, const float* esamples, int S, int n_k, int Hq, int Lq,
                            int q_pos0, double* sum, double* sumsq, int* count, double* esum, int n_rows,
                            hipStream_t s);

int launch_calibrate_rowwise(const CalibParams& p, float* samples_ws, hipStream_t s) {
    RowArgs a = {};
    a.q = p.q; a.k = p.k;
    a.B = p.S; a.Hq = p.Hq; a.Hkv = p.Hkv; a.Lq = p.Lq; a.Lk = p.Lk;
    a.xscale = p.scale * kLog2e; a.q_pos0 = p.q_pos0;
    for (int t = 0; t < 8; ++t) a.ks[t] = p.ks[t];
    a.n_k = p.n_k; a.samples = samples_ws;
    a.flags = p.pre ? kFlagPre : 0u;
    // the discarded-mass samples follow the value samples in the workspace
    float* es = p.esum ? samples_ws + (size_t)p.S * p.n_k * p.Hq * p.Lq : nullptr;
    a.esamples = es;
    int e = dispatch_rows<kRowCalib>(a, p.d, p.dtype, p.S * p.Hq * p.Lq, p.q_pos0 + p.Lq, s);
    if (e != hipSuccess) return e;
    return launch_calib_accumulate(samples_ws, es, p.S, p.n_k, p.Hq, p.Lq, p.q_pos0, p.sum, p.sumsq,
                                   p.count, p.esum, p.n_rows, s);
}

int launch_calib_accumulate(const float* samples, const float* esamples, int S, int n_k, int Hq, int Lq,
                            int q_pos0, double* sum, double* sumsq, int* count, double* esum, int n_rows,
                            hipStream_t s) {
    const size_t per = (size_t)n_k * Hq * Lq;
    hipLaunchKernelGGL(calib_accumulate_kernel, dim3((unsigned)((per + 255) / 256)), dim3(256), 0, s,
                       samples, esamples, S, n_k, Hq, Lq, q_pos0, sum, sumsq, count, esum, n_rows);
    return hipGetLastError();
}

int launch_finalize(const double* sum, const double* sumsq, const int* count, const int* ks,
                    int n_k, int Hq, int n_rows, float alpha, float* theta, hipStream_t s) {
    KList kl = {};
    for (int t = 0; t < n_k && t < 8; ++t) kl.k[t] = ks[t];
    hipLaunchKernelGGL(finalize_kernel<false>, dim3(n_k * Hq), dim3(kFinThreads), 0, s, sum, sumsq, count,
                       Hq, n_rows, kl, alpha, theta);
    return hipGetLastError();
}

int launch_finalize_etilde(const double* esum, const int* count, const int* ks, int n_k, int Hq,
                           int n_rows, float* e_tilde, hipStream_t s) {
    KList kl = {};
    for (int t = 0; t < n_k && t < 8; ++t) kl.k[t] = ks[t];
    // alpha = 0: sumsq is never read
    hipLaunchKernelGGL(finalize_kernel<true>, dim3(n_k * Hq), dim3(kFinThreads), 0, s, esum, esum, count,
                       Hq, n_rows, kl, 0.f, e_tilde);
    return hipGetLastError();
}

int launch_vmean(const void* v, const int* seq_lens, int B, int Hkv, int Lmax, int d, int dtype,
                 float* v_mean, hipStream_t s) {
    const dim3 grid(B * Hkv), block(kVmeanThreads);
    if (dtype == 0) {
        if (d == 64) hipLaunchKernelGGL((vmean_kernel<float, 64>), grid, block, 0, s, (const float*)v, seq_lens, Hkv, Lmax, v_mean);
        else hipLaunchKernelGGL((vmean_kernel<float, 128>), grid, block, 0, s, (const float*)v, seq_lens, Hkv, Lmax, v_mean);
    } else {
        if (d == 64) hipLaunchKernelGGL((vmean_kernel<uint16_t, 64>), grid, block, 0, s, (const uint16_t*)v, seq_lens, Hkv, Lmax, v_mean);
        else hipLaunchKernelGGL((vmean_kernel<uint16_t, 128>), grid, block, 0, s, (const uint16_t*)v, seq_lens, Hkv, Lmax, v_mean);
    }
    return hipGetLastError();
}

int launch_ws_prepare(void* ws, size_t header_bytes, size_t end_bytes, hipStream_t s) {
    const size_t words = end_bytes / 4;
    if (words == 0) return hipSuccess;
    unsigned blocks = (unsigned)((words + 255) / 256);
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(ws_prepare_kernel, dim3(blocks), dim3(256), 0, s, (uint32_t*)ws, header_bytes / 4, words);
    return hipGetLastError();
}

int launch_fill_u32(void* p, size_t bytes, uint32_t value, hipStream_t s) {
    const size_t words = bytes / 4;
    if (words == 0) return hipSuccess;
    unsigned blocks = (unsigned)((words + 255) / 256);
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_u32_kernel, dim3(blocks), dim3(256), 0, s, (uint32_t*)p, words, value);
    return hipGetLastError();
}

}  // namespace topth
