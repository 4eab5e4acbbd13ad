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
//      its min and max (one workgroup per sample row, scores in LDS);
//   2. sort the pooled values of each (head, row) in descending order (a
//      stable LSD radix sort of the order-preserving 32-bit keys, by one
//      workgroup, in global memory), then scan the positions, each thread
//      evaluating the condition at its own positions with binary searches in
//      the sorted sample maxima and minima, and keep for every target k the
//      smallest qualifying position (an LDS atomic min).
// Integer counts and the sort make the result exact for the values computed:
// the same values give the same theta on any launch.
#include "topth_internal.h"

#include <math.h>
#include <limits.h>

namespace topth {

constexpr int kMkcValThreads = 256;
constexpr int kMkcSelThreads = 1024;
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
    float* smin; float* smax;  // [Hq][Lq][S]
    int n_k;
    int ks[kMkcMaxTargets];
    float* theta;            // [n_k][Hq][n_rows]
};

// elements of the segments of rows 0..i-1 of one head, per sample
__host__ __device__ __forceinline__ long long mkc_row_prefix(int q_pos0, int i) {
    return (long long)i * (q_pos0 + 1) + (long long)i * (i - 1) / 2;
}

template <typename T> struct MkcLoad;
template <> struct MkcLoad<uint16_t> {   // bfloat16: 8 per 16-byte chunk
    static constexpr int EPC = 8;
    static __device__ __forceinline__ void unpack(const u32x4& u, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(u[i] << 16);
            f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    }
};
template <> struct MkcLoad<float> {
    static constexpr int EPC = 4;
    static __device__ __forceinline__ void unpack(const u32x4& u, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(u[i]);
    }
};

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
// One workgroup per (sample s, head h, row i): scores of keys 0..p into LDS
// (a group of lanes per key reads its K row in 16-byte chunks), then the
// post-softmax values s_j = exp2(x_j - lse2) (or the scores) to the pool, and
// the row's min and max.
template <typename T, int D>
__global__ __launch_bounds__(kMkcValThreads) void mkc_values_kernel(MkcArgs a) {
    extern __shared__ float s_sc[];
    __shared__ float s_red[kMkcValThreads / 64];
    constexpr int EPC = MkcLoad<T>::EPC;
    constexpr int LPR = D / EPC;               // lanes per key row
    constexpr int RPW = 64 / LPR;              // key rows per wave step
    const int row = blockIdx.x;                // ((s * Hq) + h) * Lq + i
    const int i = row % a.Lq;
    const int h = (row / a.Lq) % a.Hq;
    const int s = row / (a.Lq * a.Hq);
    const int g = a.Hq / a.Hkv;
    const int p = a.q_pos0 + i;
    const int m = p + 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % LPR, grp = lane / LPR;

    const T* qrow = (const T*)a.q + (((size_t)s * a.Hq + h) * a.Lq + i) * D;
    const T* kg = (const T*)a.k + ((size_t)s * a.Hkv + h / g) * (size_t)a.Lk * D;
    float qf[EPC];
    MkcLoad<T>::unpack(*(const u32x4*)(qrow + sub * EPC), qf);

    float mx = -INFINITY;
    for (int j0 = wave * RPW; j0 < m; j0 += (kMkcValThreads / 64) * RPW) {
        const int j = j0 + grp;
        float dot = 0.f;
        if (j < m) {
            float kf[EPC];
            MkcLoad<T>::unpack(*(const u32x4*)(kg + (size_t)j * D + sub * EPC), kf);
#pragma unroll
            for (int e = 0; e < EPC; ++e) dot = fmaf(qf[e], kf[e], dot);
        }
#pragma unroll
        for (int o = 1; o < LPR; o <<= 1) dot += __shfl_xor(dot, o);
        if (j < m && sub == 0) {
            const float x = a.pre ? dot * a.scale : dot * a.xscale;
            s_sc[j] = x;
            mx = fmaxf(mx, x);
        }
    }
    mx = block_reduce(mx, s_red, true);        // its barriers also publish s_sc
    float out_min = INFINITY, out_max = -INFINITY;
    float* dst = a.pool + (size_t)h * a.S * mkc_row_prefix(a.q_pos0, a.Lq) +
                 (size_t)a.S * mkc_row_prefix(a.q_pos0, i) + (size_t)s * m;
    if (a.pre) {
        for (int j = threadIdx.x; j < m; j += kMkcValThreads) {
            const float v = s_sc[j] + 0.0f;    // -0 becomes +0: one key per value
            dst[j] = v;
            out_min = fminf(out_min, v);
            out_max = fmaxf(out_max, v);
        }
    } else {
        float l = 0.f;
        for (int j = threadIdx.x; j < m; j += kMkcValThreads) l += exp2f(s_sc[j] - mx);
        l = block_reduce(l, s_red, false);
        const float lse2 = mx + log2f(l);
        for (int j = threadIdx.x; j < m; j += kMkcValThreads) {
            const float v = exp2f(s_sc[j] - lse2);
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

// One workgroup of 1024 threads per (head h, row i).
__global__ __launch_bounds__(kMkcSelThreads) void mkc_select_kernel(MkcArgs a) {
    __shared__ float s_max[kMkcMaxSamples], s_min[kMkcMaxSamples];
    __shared__ int s_hist[256], s_base[256], s_tile[256];
    __shared__ int s_cnt[kMkcSelThreads / 64][256];
    __shared__ int s_best[kMkcMaxTargets];
    constexpr int NW = kMkcSelThreads / 64;
    const int seg = blockIdx.x;                // h * Lq + i
    const int i = seg % a.Lq, h = seg / a.Lq;
    const int p = a.q_pos0 + i;
    const int m = p + 1;
    const int S = a.S;
    const int N = S * m;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t off = (size_t)h * S * mkc_row_prefix(a.q_pos0, a.Lq) + (size_t)S * mkc_row_prefix(a.q_pos0, i);
    float* src = a.pool + off;
    float* dst = a.pool2 + off;

    // sample maxima and minima, ascending, padded with -inf to a power of two
    int n2 = 1;
    while (n2 < S) n2 <<= 1;
    for (int c = tid; c < n2; c += kMkcSelThreads) {
        const size_t o = ((size_t)h * a.Lq + i) * S + c;
        s_max[c] = c < S ? a.smax[o] : -INFINITY;
        s_min[c] = c < S ? a.smin[o] : -INFINITY;
    }
    for (int t = tid; t < kMkcMaxTargets; t += kMkcSelThreads) s_best[t] = INT_MAX;
    for (int t = tid; t < NW * 256; t += kMkcSelThreads) (&s_cnt[0][0])[t] = 0;
    lds_bitonic_asc(s_max, n2);
    lds_bitonic_asc(s_min, n2);

    // stable LSD radix sort, 8 bits per pass, of the keys of the N values
    const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int sh = 0; sh < 32; sh += 8) {
        for (int t = tid; t < 256; t += kMkcSelThreads) s_hist[t] = 0;
        __syncthreads();
        for (int j = tid; j < N; j += kMkcSelThreads)
            atomicAdd(&s_hist[(mkc_key(src[j]) >> sh) & 255u], 1);
        __syncthreads();
        if (tid < 64) {                        // exclusive scan of the 256 bins, 4 per lane
            int v[4], sum = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) { v[e] = s_hist[4 * tid + e]; sum += v[e]; }
            int incl = sum;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int w = __shfl_up(incl, o);
                if (lane >= o) incl += w;
            }
            int run = incl - sum;
#pragma unroll
            for (int e = 0; e < 4; ++e) { s_base[4 * tid + e] = run; run += v[e]; }
        }
        __syncthreads();
        for (int t0 = 0; t0 < N; t0 += kMkcSelThreads) {
            const int j = t0 + tid;
            const bool valid = j < N;
            const float v = valid ? src[j] : 0.f;
            const int dg = valid ? (int)((mkc_key(v) >> sh) & 255u) : 0;
            // lanes of this wave with the same digit, in lane order
            unsigned long long peers = __ballot(valid);
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const unsigned long long bb = __ballot(valid && ((dg >> b) & 1));
                peers &= ((dg >> b) & 1) ? bb : ~bb;
            }
            const int rank = __popcll(peers & lt);
            if (valid && rank == 0) s_cnt[wave][dg] = __popcll(peers);
            __syncthreads();
            if (tid < 256) {                   // prefix over the waves, per digit
                int run = 0;
#pragma unroll
                for (int w = 0; w < NW; ++w) { const int c = s_cnt[w][tid]; s_cnt[w][tid] = run; run += c; }
                s_tile[tid] = run;
            }
            __syncthreads();
            if (valid) dst[s_base[dg] + s_cnt[wave][dg] + rank] = v;
            __syncthreads();
            if (tid < 256) {
                s_base[tid] += s_tile[tid];
#pragma unroll
                for (int w = 0; w < NW; ++w) s_cnt[w][tid] = 0;
            }
            __syncthreads();
        }
        float* t = src; src = dst; dst = t;    // the sorted pass is the next source
    }
    // after four passes the values are back in the first buffer, descending

    // the walk: every position that ends a run of equal values
    for (int j = tid; j < N; j += kMkcSelThreads) {
        const float x = src[j];
        if (j + 1 < N && src[j + 1] == x) continue;
        const int Mx = count_ge(s_max, n2, x);
        const int Nl = count_ge(s_min, n2, x);
        const long long C = (long long)Mx - Nl;
        if (C <= 0) continue;
        const long long T = (long long)(j + 1) - (long long)m * Nl;
        for (int t = 0; t < a.n_k; ++t)
            if (T >= (long long)a.ks[t] * C) atomicMin(&s_best[t], j);
    }
    __syncthreads();
    if (p < a.n_rows)
        for (int t = tid; t < a.n_k; t += kMkcSelThreads) {
            const int b = s_best[t];
            a.theta[((size_t)t * a.Hq + h) * a.n_rows + p] = b == INT_MAX ? -INFINITY : src[b];
        }
}

// ------------------------------------------------------------------ host side
size_t mkc_ws_bytes(int S, int Hq, int Lq, int Lk) {
    const size_t seg = (size_t)S * Hq * Lq * Lk;          // bound of the pooled values
    return 2 * seg * sizeof(float) + 2 * (size_t)Hq * Lq * S * sizeof(float) + 1024;
}

int mkc_max_samples() { return kMkcMaxSamples; }
int mkc_max_targets() { return kMkcMaxTargets; }
int mkc_max_keys() { return kMkcMaxKeys; }

template <typename T, int D>
static int launch_values(const MkcArgs& a, hipStream_t s) {
    const int m_max = a.q_pos0 + a.Lq;
    const size_t smem = (size_t)m_max * sizeof(float);
    if (smem > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)mkc_values_kernel<T, D>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((mkc_values_kernel<T, D>), dim3(a.S * a.Hq * a.Lq), dim3(kMkcValThreads), smem, s, a);
    return hipGetLastError();
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
    a.n_k = p.n_k;
    for (int t = 0; t < p.n_k; ++t) a.ks[t] = p.mkc_ks[t];
    a.theta = theta;
    int e;
    if (p.dtype == 1) e = p.d == 64 ? launch_values<uint16_t, 64>(a, s) : launch_values<uint16_t, 128>(a, s);
    else e = p.d == 64 ? launch_values<float, 64>(a, s) : launch_values<float, 128>(a, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(mkc_select_kernel, dim3(p.Hq * p.Lq), dim3(kMkcSelThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace topth
