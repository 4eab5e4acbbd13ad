// Decode-serving helpers around Top-theta ("Top-Theta Attention: Sparsifying
// Transformers by Compensated Thresholding"):
//   * the running mean of V that VMC adds (Sec. 3.2.2, after Eq. 7: during
//     generative decoding mu is kept as a running mean), updated when rows are
//     appended to a KV cache;
//   * thresholds for rows no calibration reached, from a least-squares fit of
//     the calibrated rows as a function of the row position (the paper fits
//     thresholds to the sequence length; the function is not given, so a low
//     degree polynomial in ln(p + 1) is used: on ln(theta) for post-softmax
//     thresholds, on theta for pre-softmax ones).
// These run once per appended token or once per calibration, not per score
// element; they are written for determinism (fixed summation order, float64)
// rather than speed.
#include "topth_internal.h"

#include <math.h>

namespace topth {

// mu over the first n_new rows from mu over the first n_old rows: one
// workgroup per (b, KV head); each thread sums 16-byte pieces of the appended
// rows in float64 in row order, the partial sums are added in a fixed order.
constexpr int kAppendThreads = 256;
template <typename T, int D>
__global__ __launch_bounds__(kAppendThreads) void vmean_append_kernel(
        const T* v, const int* old_lens, const int* new_lens, int Hkv, int Lmax, float* mu) {
    constexpr int EPC = 16 / (int)sizeof(T);          // elements per 16-byte piece
    constexpr int CPR = D / EPC;                      // pieces per row
    constexpr int RS = kAppendThreads / CPR;          // rows per pass
    __shared__ double part[RS][D];
    const int bk = blockIdx.x;
    const int b = bk / Hkv;
    const int n_new = min(max(new_lens[b], 1), Lmax);
    const int n_old = old_lens ? min(max(old_lens[b], 0), n_new) : n_new - 1;   // NULL: one row appended
    const T* base = v + (size_t)bk * Lmax * D;
    const int c = threadIdx.x % CPR, r0 = threadIdx.x / CPR;
    double acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.0;
    for (int j = n_old + r0; j < n_new; j += RS) {
        const u32x4 raw = *(const u32x4*)(base + (size_t)j * D + c * EPC);
        const T* x = reinterpret_cast<const T*>(&raw);
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[e] += (double)Elem<T>::load(x + e);
    }
#pragma unroll
    for (int e = 0; e < EPC; ++e) part[r0][c * EPC + e] = acc[e];
    __syncthreads();
    for (int t = threadIdx.x; t < D; t += kAppendThreads) {
        double sum = n_old > 0 ? (double)n_old * (double)mu[(size_t)bk * D + t] : 0.0;
        for (int r = 0; r < RS; ++r) sum += part[r][t];
        mu[(size_t)bk * D + t] = (float)(sum / (double)n_new);
    }
}

// Least-squares polynomial fit per (k, head): normal equations in float64
// over the observed rows (count > 0, theta finite, and theta > 0 in the log
// domain), solved by Gaussian elimination with partial pivoting.  Coefficients
// are stored highest power first; NaN when fewer than degree + 1 rows are
// usable or the system is singular.
constexpr int kFitThreads = 256;
constexpr int kMaxFitDegree = 3;
struct FitKList { int k[8]; };
__global__ __launch_bounds__(kFitThreads) void theta_fit_kernel(
        const float* theta, const int* count, FitKList p_min, int Hq, int n_rows, int degree, int log_domain,
        double* coef) {
    constexpr int NS = 2 * kMaxFitDegree + 1;          // power sums x^0 .. x^(2 deg)
    constexpr int NT = kMaxFitDegree + 1;              // moments x^0 y .. x^deg y
    __shared__ double s_pow[kFitThreads][NS + NT + 1];
    const size_t base = (size_t)blockIdx.x * n_rows;
    double sp[NS + NT + 1];
#pragma unroll
    for (int i = 0; i < NS + NT + 1; ++i) sp[i] = 0.0;
    for (int p = p_min.k[blockIdx.x / Hq] + threadIdx.x; p < n_rows; p += kFitThreads) {
        if (count[base + p] <= 0) continue;
        const float th = theta[base + p];
        if (!isfinite(th) || (log_domain && !(th > 0.0f))) continue;
        const double x = log((double)p + 1.0);
        const double y = log_domain ? log((double)th) : (double)th;
        double xp = 1.0;
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            if (i <= 2 * degree) sp[i] += xp;
            if (i < NT && i <= degree) sp[NS + (i < NT ? i : 0)] += xp * y;
            xp *= x;
        }
        sp[NS + NT] += 1.0;                            // usable rows
    }
#pragma unroll
    for (int i = 0; i < NS + NT + 1; ++i) s_pow[threadIdx.x][i] = sp[i];
    __syncthreads();
    if (threadIdx.x != 0) return;
    double tot[NS + NT + 1];
    for (int i = 0; i < NS + NT + 1; ++i) {
        double s = 0.0;
        for (int t = 0; t < kFitThreads; ++t) s += s_pow[t][i];
        tot[i] = s;
    }
    const int m = degree + 1;
    double* out = coef + (size_t)blockIdx.x * m;
    if (tot[NS + NT] < (double)m) {
        for (int i = 0; i < m; ++i) out[i] = NAN;
        return;
    }
    // A[i][j] = sum x^(i+j), rhs[i] = sum x^i y, unknowns c_j of x^j
    double A[NT][NT + 1];
    for (int i = 0; i < m; ++i) {
        for (int j = 0; j < m; ++j) A[i][j] = tot[i + j];
        A[i][m] = tot[NS + i];
    }
    for (int col = 0; col < m; ++col) {
        int piv = col;
        for (int r = col + 1; r < m; ++r)
            if (fabs(A[r][col]) > fabs(A[piv][col])) piv = r;
        if (!(fabs(A[piv][col]) > 1e-300)) {
            for (int i = 0; i < m; ++i) out[i] = NAN;
            return;
        }
        if (piv != col)
            for (int j = 0; j <= m; ++j) { const double t = A[col][j]; A[col][j] = A[piv][j]; A[piv][j] = t; }
        for (int r = col + 1; r < m; ++r) {
            const double f = A[r][col] / A[col][col];
            for (int j = col; j <= m; ++j) A[r][j] -= f * A[col][j];
        }
    }
    double c[NT];
    for (int i = m - 1; i >= 0; --i) {
        double s = A[i][m];
        for (int j = i + 1; j < m; ++j) s -= A[i][j] * c[j];
        c[i] = s / A[i][i];
    }
    for (int i = 0; i < m; ++i) out[i] = c[m - 1 - i];   // highest power first
}

// theta_out[t][h][p] = the fitted polynomial at ln(p + 1) (exponentiated in
// the log domain) for p + 1 > k, -inf for rows that keep every element.
__global__ void theta_eval_kernel(const double* coef, FitKList ks, int Hq, int degree, int log_domain,
                                  int n_out, float* theta_out) {
    const int th = blockIdx.y;                         // t * Hq + h
    const int p = blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= n_out) return;
    const int k = ks.k[th / Hq];
    float v = -INFINITY;
    if (p + 1 > k) {
        const double* c = coef + (size_t)th * (degree + 1);
        const double x = log((double)p + 1.0);
        double y = c[0];
        for (int i = 1; i <= degree; ++i) y = y * x + c[i];
        v = (float)(log_domain ? exp(y) : y);
    }
    theta_out[(size_t)th * n_out + p] = v;
}

// ------------------------------------------------------------------ host side
int max_fit_degree() { return kMaxFitDegree; }

int launch_vmean_append(const void* v, const int* old_lens, const int* new_lens, int B, int Hkv, int Lmax,
                        int d, int dtype, float* v_mean, hipStream_t s) {
    const dim3 grid(B * Hkv), block(kAppendThreads);
    if (dtype == 0) {
        if (d == 64) hipLaunchKernelGGL((vmean_append_kernel<float, 64>), grid, block, 0, s, (const float*)v, old_lens, new_lens, Hkv, Lmax, v_mean);
        else hipLaunchKernelGGL((vmean_append_kernel<float, 128>), grid, block, 0, s, (const float*)v, old_lens, new_lens, Hkv, Lmax, v_mean);
    } else {
        if (d == 64) hipLaunchKernelGGL((vmean_append_kernel<uint16_t, 64>), grid, block, 0, s, (const uint16_t*)v, old_lens, new_lens, Hkv, Lmax, v_mean);
        else hipLaunchKernelGGL((vmean_append_kernel<uint16_t, 128>), grid, block, 0, s, (const uint16_t*)v, old_lens, new_lens, Hkv, Lmax, v_mean);
    }
    return hipGetLastError();
}

int launch_theta_fit(const float* theta, const int* count, const int* ks, int n_k, int Hq, int n_rows,
                     int degree, int log_domain, int min_len_over_k, double* coef, hipStream_t s) {
    FitKList p_min = {};                               // first row of the fit, per k
    for (int t = 0; t < n_k && t < 8; ++t) {
        const long long r = (long long)min_len_over_k * ks[t] - 1;
        p_min.k[t] = r < 0 ? 0 : (r > n_rows ? n_rows : (int)r);
    }
    hipLaunchKernelGGL(theta_fit_kernel, dim3(n_k * Hq), dim3(kFitThreads), 0, s, theta, count, p_min, Hq,
                       n_rows, degree, log_domain, coef);
    return hipGetLastError();
}

int launch_theta_eval(const double* coef, const int* ks, int n_k, int Hq, int degree, int log_domain,
                      int n_out, float* theta_out, hipStream_t s) {
    FitKList kl = {};
    for (int t = 0; t < n_k && t < 8; ++t) kl.k[t] = ks[t];
    const dim3 grid((n_out + 255) / 256, n_k * Hq);
    hipLaunchKernelGGL(theta_eval_kernel, grid, dim3(256), 0, s, coef, kl, Hq, degree, log_domain, n_out,
                       theta_out);
    return hipGetLastError();
}

}  // namespace topth
