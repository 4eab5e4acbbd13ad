// C ABI of libtopth: argument validation, workspace sizing and dispatch.
// Every argument error is reported before anything is enqueued on the stream;
// no C++ exception leaves this file.
#include "topth.h"
#include "topth_internal.h"

#include <math.h>
#include <limits.h>

namespace topth {
// defined in the kernel sources
bool decode_bf16_supported(int d, int G);
int launch_decode_bf16(const DecodeParams& p, hipStream_t s);
int launch_decode_bf16_noalloc(DecodeParams p, bool* fits, hipStream_t s);
int noalloc_scratch(void** out);
size_t noalloc_scratch_bytes();
int launch_decode_rowwise(const DecodeParams& p, uint32_t* masks_ws, hipStream_t s);
size_t decode_rowwise_ws_bytes(int B, int Hq, int Lmax);
int rowwise_max_keys();
int launch_prefill_rowwise(const PrefillParams& p, float* mu_ws, hipStream_t s);
bool prefill_bf16_supported(int d, int G);
int launch_prefill_bf16(const PrefillParams& p, float* mu_ws, hipStream_t s);
int launch_calibrate_rowwise(const CalibParams& p, float* samples_ws, hipStream_t s);
bool calib_bf16_supported(int d, int S, int Hq, int Lq, int q_pos0);
int launch_calibrate_bf16(const CalibParams& p, float* samples_ws, hipStream_t s);
int max_fit_degree();
size_t mkc_ws_bytes(int S, int Hq, int Lq, int Lk);
int mkc_max_samples();
int mkc_max_targets();
int mkc_max_keys();
int launch_calibrate_mkc(const CalibParams& p, int pre, float* theta, hipStream_t s);
int launch_vmean_append(const void* v, const int* old_lens, const int* new_lens, int B, int Hkv, int Lmax,
                        int d, int dtype, float* v_mean, hipStream_t s);
int launch_theta_fit(const float* theta, const int* count, const int* ks, int n_k, int Hq, int n_rows,
                     int degree, int log_domain, int min_len_over_k, double* coef, hipStream_t s);
int launch_theta_eval(const double* coef, const int* ks, int n_k, int Hq, int degree, int log_domain,
                      int n_out, float* theta_out, hipStream_t s);
}  // namespace topth

using namespace topth;

static_assert(kNoallocScratchBytes == (size_t)TOPTH_NOALLOC_SCRATCH_BYTES, "scratch size of the header");
static_assert(kFlagOutF32 == TOPTH_OUT_F32 && kFlagVmc == TOPTH_VMC && kFlagNone == TOPTH_SDC_NONE &&
                  kFlagExpth == TOPTH_SDC_EXPTH && kFlagOffline == TOPTH_SDC_OFFLINE, "flag bits of the header");
static_assert(kWsHeaderBytes == TOPTH_WS_HEADER_BYTES && kStatusSpinTimeout == TOPTH_STATUS_EXCHANGE_TIMEOUT,
              "workspace header layout of the header");

namespace {

bool bad_dims(int B, int Hq, int Hkv, int L, int d) {
    return B <= 0 || Hq <= 0 || Hkv <= 0 || L <= 0 || (Hq % Hkv) != 0 || (d != 64 && d != 128);
}

bool bad_dtype(int dtype) { return dtype != TOPTH_F32 && dtype != TOPTH_BF16; }

// elements of a [a][b][c][d] tensor fit comfortably in size_t and in the
// 32-bit row indices the kernels use for rows
bool too_big(long long rows, long long cols) {
    return rows <= 0 || cols <= 0 || rows > (long long)INT_MAX || rows * cols > (1LL << 40);
}

int map_hip(int e) { return e == 0 ? TOPTH_OK : TOPTH_EHIP; }

// prefix means of V (VMC), then a float16 copy of V (transposed 64-key tiles)
// and a flag word (bf16 P V in float16); a workspace with only the first part
// still serves VMC
size_t prefill_ws_vmc(int B, int Hkv, int L, int d) {
    return (size_t)B * Hkv * L * d * sizeof(float) + 256;
}
size_t prefill_ws(int B, int Hq, int Hkv, int L, int d) {
    (void)Hq;
    const size_t mu = ((size_t)B * Hkv * L * d * sizeof(float) + 255) & ~(size_t)255;
    const size_t v16 = ((size_t)B * Hkv * (size_t)((L + 63) / 64) * 64 * d * sizeof(uint16_t) + 255) & ~(size_t)255;
    return mu + v16 + 256;
}

// per-sequence samples; then, for the tiled kernel, a counter and a list of
// (row, target) entries for the exact fixup (at most one per sample)
size_t calib_ws(int S, int Hq, int Lq, int n_k) {
    const size_t n = (size_t)S * n_k * Hq * Lq;
    return ((n * sizeof(float) + 255) & ~(size_t)255) + 256 + n * 16 + 256;
}

// flags of the pre-softmax calls: VMC plus at most one estimate of E~
bool bad_pre_flags(unsigned flags, const float* e_tilde, float gamma) {
    if (flags & ~(TOPTH_VMC | TOPTH_SDC_NONE | TOPTH_SDC_EXPTH | TOPTH_SDC_OFFLINE)) return true;
    const unsigned est = flags & (TOPTH_SDC_NONE | TOPTH_SDC_EXPTH | TOPTH_SDC_OFFLINE);
    if (est & (est - 1)) return true;                         // more than one estimate
    if ((flags & TOPTH_SDC_OFFLINE) && !e_tilde) return true;
    if ((flags & TOPTH_SDC_EXPTH) && !(isfinite(gamma) && gamma >= 0.0f)) return true;
    return false;
}

size_t decode_ws(int B, int Hq, int Hkv, int Lmax, int d) {
    size_t a = decode_ws_bytes(B, Hq, Hkv, Lmax, d);
    size_t b = kWsHeaderBytes + decode_rowwise_ws_bytes(B, Hq, Lmax) + 256;
    return a > b ? a : b;
}

}  // namespace

extern "C" {

const char* topth_strerror(int status) {
    switch (status) {
        case TOPTH_OK: return "success";
        case TOPTH_EINVAL: return "invalid argument";
        case TOPTH_EUNSUPPORTED: return "unsupported shape or type";
        case TOPTH_EWORKSPACE: return "workspace missing or too small";
        case TOPTH_EHIP: return "HIP runtime error";
        case TOPTH_ESCRATCH: return "shape needs more scratch than the library's static device buffer holds";
        default: return "unknown status";
    }
}

size_t topth_workspace_size(int op, int B, int Hq, int Hkv, int Lq, int Lk, int d, int n_k) {
    switch (op) {
        case TOPTH_OP_CALIBRATE:
            if (bad_dims(B, Hq, Hkv, Lq, d) || Lk <= 0 || n_k < 1 || n_k > TOPTH_MAX_NK) return 0;
            return calib_ws(B, Hq, Lq, n_k);
        case TOPTH_OP_CALIBRATE_PRE_E:   // value samples, then discarded-mass samples
            if (bad_dims(B, Hq, Hkv, Lq, d) || Lk <= 0 || n_k < 1 || n_k > TOPTH_MAX_NK) return 0;
            return 2 * calib_ws(B, Hq, Lq, n_k);
        case TOPTH_OP_PREFILL:
            if (bad_dims(B, Hq, Hkv, Lq, d)) return 0;
            return prefill_ws(B, Hq, Hkv, Lq, d);
        case TOPTH_OP_DECODE:
            if (bad_dims(B, Hq, Hkv, Lk, d)) return 0;
            return decode_ws(B, Hq, Hkv, Lk, d);
        case TOPTH_OP_CALIBRATE_MKC:
            if (bad_dims(B, Hq, Hkv, Lq, d) || Lk <= 0 || Lq > Lk || B > mkc_max_samples() || Lk > mkc_max_keys())
                return 0;
            return mkc_ws_bytes(B, Hq, Lq, Lk);
        default:
            return 0;
    }
}

int topth_workspace_init(void* ws, size_t ws_bytes, void* stream) {
    if (!ws || ws_bytes == 0) return TOPTH_EINVAL;
    // header zero (status word), every slot after it empty
    const size_t head = ws_bytes < kWsHeaderBytes ? ws_bytes : kWsHeaderBytes;
    int e = launch_fill_u32(ws, head, 0u, (hipStream_t)stream);
    if (e == hipSuccess && ws_bytes > kWsHeaderBytes)
        e = launch_fill_u32((char*)ws + kWsHeaderBytes, ws_bytes - kWsHeaderBytes, kWsSlotEmpty,
                            (hipStream_t)stream);
    return map_hip(e);
}

int topth_workspace_status(const void* ws, size_t ws_bytes, int* status, void* stream) {
    if (!ws || !status || ws_bytes < kWsHeaderBytes) return TOPTH_EINVAL;
    int word = 0;
    hipError_t e = hipMemcpyAsync(&word, ws, sizeof(int), hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return TOPTH_EHIP;
    *status = word;
    return TOPTH_OK;
}

int topth_workspace_set_spin_limit(void* ws, size_t ws_bytes, unsigned limit, void* stream) {
    if (!ws || ws_bytes < kWsHeaderBytes) return TOPTH_EINVAL;
    return map_hip(launch_fill_u32((char*)ws + 4, 4, limit, (hipStream_t)stream));
}

}  // extern "C"

namespace {

int calibrate_common(const void* q, const void* k, int S, int Hq, int Hkv, int Lq, int Lk,
                     int d, int dtype, float scale, int q_pos0, const int* ks, int n_k,
                     double* sum, double* sumsq, int* count, int n_rows,
                     void* ws, size_t ws_bytes, void* stream, bool pre, double* esum) {
    if (!q || !k || !ks || !sum || !sumsq || !count) return TOPTH_EINVAL;
    if (bad_dims(S, Hq, Hkv, Lq, d) || bad_dtype(dtype) || Lk <= 0 || n_rows <= 0) return TOPTH_EINVAL;
    if (!isfinite(scale) || !(scale > 0.0f) || q_pos0 < 0 || q_pos0 + Lq > Lk) return TOPTH_EINVAL;
    if (n_k < 1 || n_k > TOPTH_MAX_NK) return TOPTH_EINVAL;
    for (int t = 0; t < n_k; ++t)
        if (ks[t] < 1) return TOPTH_EINVAL;
    if (too_big((long long)S * Hq * Lq, d) || too_big((long long)S * Hkv * Lk, d)) return TOPTH_EUNSUPPORTED;
    const bool tiled = dtype == TOPTH_BF16 && calib_bf16_supported(d, S, Hq, Lq, q_pos0);
    if (!tiled && Lk > rowwise_max_keys()) return TOPTH_EUNSUPPORTED;
    if (!ws) return TOPTH_EWORKSPACE;
    const size_t need = (esum ? 2 : 1) * calib_ws(S, Hq, Lq, n_k);
    if (ws_bytes < need) return TOPTH_EWORKSPACE;
    CalibParams p = {};
    p.q = q; p.k = k; p.S = S; p.Hq = Hq; p.Hkv = Hkv; p.Lq = Lq; p.Lk = Lk; p.d = d;
    p.dtype = dtype; p.scale = scale; p.q_pos0 = q_pos0;
    for (int t = 0; t < n_k; ++t) p.ks[t] = ks[t];
    p.n_k = n_k; p.sum = sum; p.sumsq = sumsq; p.count = count; p.n_rows = n_rows;
    p.ws = ws; p.ws_bytes = ws_bytes;
    p.pre = pre; p.esum = esum;
    return map_hip(tiled ? launch_calibrate_bf16(p, (float*)ws, (hipStream_t)stream)
                         : launch_calibrate_rowwise(p, (float*)ws, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int topth_calibrate(const void* q, const void* k, int S, int Hq, int Hkv, int Lq, int Lk,
                    int d, int dtype, float scale, int q_pos0, const int* ks, int n_k,
                    double* sum, double* sumsq, int* count, int n_rows,
                    void* ws, size_t ws_bytes, void* stream) {
    return calibrate_common(q, k, S, Hq, Hkv, Lq, Lk, d, dtype, scale, q_pos0, ks, n_k, sum, sumsq,
                            count, n_rows, ws, ws_bytes, stream, false, nullptr);
}

int topth_calibrate_pre(const void* q, const void* k, int S, int Hq, int Hkv, int Lq, int Lk,
                        int d, int dtype, float scale, int q_pos0, const int* ks, int n_k,
                        double* sum, double* sumsq, int* count, double* esum, int n_rows,
                        void* ws, size_t ws_bytes, void* stream) {
    return calibrate_common(q, k, S, Hq, Hkv, Lq, Lk, d, dtype, scale, q_pos0, ks, n_k, sum, sumsq,
                            count, n_rows, ws, ws_bytes, stream, true, esum);
}

int topth_calibrate_mkc(const void* q, const void* k, int S, int Hq, int Hkv, int Lq, int Lk, int d,
                        int dtype, float scale, int q_pos0, int pre, const int* ks, int n_k,
                        float* theta, int n_rows, void* ws, size_t ws_bytes, void* stream) {
    if (!q || !k || !ks || !theta) return TOPTH_EINVAL;
    if (bad_dims(S, Hq, Hkv, Lq, d) || bad_dtype(dtype) || Lk <= 0 || n_rows <= 0) return TOPTH_EINVAL;
    if (!isfinite(scale) || !(scale > 0.0f) || q_pos0 < 0 || q_pos0 + Lq > Lk) return TOPTH_EINVAL;
    if (pre != 0 && pre != 1) return TOPTH_EINVAL;
    if (n_k < 1 || n_k > mkc_max_targets()) return TOPTH_EINVAL;
    for (int t = 0; t < n_k; ++t)
        if (ks[t] < 1) return TOPTH_EINVAL;
    if (S > mkc_max_samples() || Lk > mkc_max_keys()) return TOPTH_EUNSUPPORTED;
    if ((long long)S * Hq * Lq > INT_MAX || (long long)Hq * Lq > INT_MAX) return TOPTH_EUNSUPPORTED;
    if (!ws) return TOPTH_EWORKSPACE;
    if (ws_bytes < mkc_ws_bytes(S, Hq, Lq, Lk)) return TOPTH_EWORKSPACE;
    CalibParams p = {};
    p.q = q; p.k = k; p.S = S; p.Hq = Hq; p.Hkv = Hkv; p.Lq = Lq; p.Lk = Lk; p.d = d;
    p.dtype = dtype; p.scale = scale; p.q_pos0 = q_pos0; p.n_k = n_k; p.mkc_ks = ks;
    p.n_rows = n_rows; p.ws = ws; p.ws_bytes = ws_bytes;
    return map_hip(launch_calibrate_mkc(p, pre, theta, (hipStream_t)stream));
}

int topth_calibrate_finalize_etilde(const double* esum, const int* count, const int* ks, int n_k,
                                    int Hq, int n_rows, float* e_tilde, void* stream) {
    if (!esum || !count || !ks || !e_tilde) return TOPTH_EINVAL;
    if (n_k < 1 || n_k > TOPTH_MAX_NK || Hq <= 0 || n_rows <= 0) return TOPTH_EINVAL;
    if ((float)n_rows > 16777216.0f) return TOPTH_EUNSUPPORTED;
    for (int t = 0; t < n_k; ++t)
        if (ks[t] < 1) return TOPTH_EINVAL;
    return map_hip(launch_finalize_etilde(esum, count, ks, n_k, Hq, n_rows, e_tilde, (hipStream_t)stream));
}

int topth_calibrate_finalize(const double* sum, const double* sumsq, const int* count,
                             const int* ks, int n_k, int Hq, int n_rows, float alpha,
                             float* theta, void* stream) {
    if (!sum || !sumsq || !count || !ks || !theta) return TOPTH_EINVAL;
    if (n_k < 1 || n_k > TOPTH_MAX_NK || Hq <= 0 || n_rows <= 0 || !isfinite(alpha)) return TOPTH_EINVAL;
    if ((float)n_rows > 16777216.0f) return TOPTH_EUNSUPPORTED;
    for (int t = 0; t < n_k; ++t)
        if (ks[t] < 1) return TOPTH_EINVAL;
    return map_hip(launch_finalize(sum, sumsq, count, ks, n_k, Hq, n_rows, alpha, theta,
                                   (hipStream_t)stream));
}

}  // extern "C"

namespace {

int prefill_common(const void* q, const void* k, const void* v, int B, int Hq, int Hkv, int L,
                   int d, int dtype, float scale, const float* theta, int n_rows,
                   unsigned flags, void* out, int* kept_count, float* beta,
                   unsigned char* kept_mask, void* ws, size_t ws_bytes, void* stream,
                   bool pre, const float* e_tilde, float gamma) {
    if (!q || !k || !v || !theta || !out) return TOPTH_EINVAL;
    if (bad_dims(B, Hq, Hkv, L, d) || bad_dtype(dtype) || n_rows <= 0) return TOPTH_EINVAL;
    if (!isfinite(scale) || !(scale > 0.0f)) return TOPTH_EINVAL;
    const unsigned out_f32 = (flags & TOPTH_OUT_F32) && dtype == TOPTH_BF16 ? kFlagOutF32 : 0u;
    flags &= ~TOPTH_OUT_F32;
    if (pre ? bad_pre_flags(flags, e_tilde, gamma) : (flags & ~(TOPTH_VMC | TOPTH_SDC_NONE)) != 0)
        return TOPTH_EINVAL;
    if (too_big((long long)B * Hq * L, d)) return TOPTH_EUNSUPPORTED;
    if (dtype == TOPTH_F32 && L > rowwise_max_keys()) return TOPTH_EUNSUPPORTED;
    if (dtype == TOPTH_BF16 && (!prefill_bf16_supported(d, Hq / Hkv) || (long long)L * d * 2 >= INT_MAX))
        return TOPTH_EUNSUPPORTED;
    const bool vmc = (flags & TOPTH_VMC) && !(flags & TOPTH_SDC_NONE);
    if (vmc) {
        if (!ws) return TOPTH_EWORKSPACE;
        if (ws_bytes < prefill_ws_vmc(B, Hkv, L, d)) return TOPTH_EWORKSPACE;
    }
    PrefillParams p = {};
    p.q = q; p.k = k; p.v = v; p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.L = L; p.d = d; p.dtype = dtype;
    p.scale = scale; p.theta = theta; p.n_rows = n_rows; p.flags = flags | out_f32;
    p.out = out; p.kept_count = kept_count; p.beta = beta; p.kept_mask = kept_mask;
    p.ws = ws; p.ws_bytes = ws_bytes;
    if (pre) { p.flags |= kFlagPre; p.e_tilde = e_tilde; p.gamma = gamma; }
    if (dtype == TOPTH_BF16) return map_hip(launch_prefill_bf16(p, (float*)ws, (hipStream_t)stream));
    return map_hip(launch_prefill_rowwise(p, (float*)ws, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int topth_prefill(const void* q, const void* k, const void* v, int B, int Hq, int Hkv, int L,
                  int d, int dtype, float scale, const float* theta, int n_rows,
                  unsigned flags, void* out, int* kept_count, float* beta,
                  unsigned char* kept_mask, void* ws, size_t ws_bytes, void* stream) {
    return prefill_common(q, k, v, B, Hq, Hkv, L, d, dtype, scale, theta, n_rows, flags, out,
                          kept_count, beta, kept_mask, ws, ws_bytes, stream, false, nullptr, 0.f);
}

int topth_prefill_pre(const void* q, const void* k, const void* v, int B, int Hq, int Hkv, int L,
                      int d, int dtype, float scale, const float* theta, const float* e_tilde,
                      int n_rows, unsigned flags, float gamma, void* out, int* kept_count,
                      float* beta, unsigned char* kept_mask, void* ws, size_t ws_bytes, void* stream) {
    return prefill_common(q, k, v, B, Hq, Hkv, L, d, dtype, scale, theta, n_rows, flags, out,
                          kept_count, beta, kept_mask, ws, ws_bytes, stream, true, e_tilde, gamma);
}

}  // extern "C"

namespace {

int decode_common(const void* q, const void* k_cache, const void* v_cache, const int* seq_lens,
                  int B, int Hq, int Hkv, int Lmax, int d, int dtype, float scale,
                  const float* theta, int n_rows, const float* v_mean, unsigned flags,
                  void* out, int* kept_count, float* beta, int* vrows_read,
                  unsigned char* kept_mask, void* ws, size_t ws_bytes, void* stream,
                  bool pre, const float* e_tilde, float gamma, int min_votes = 1, int augment = 0,
                  float* v_mean_append = nullptr) {
    if (!q || !k_cache || !v_cache || !seq_lens || !theta || !out) return TOPTH_EINVAL;
    if (bad_dims(B, Hq, Hkv, Lmax, d) || bad_dtype(dtype) || n_rows <= 0) return TOPTH_EINVAL;
    if (!isfinite(scale) || !(scale > 0.0f)) return TOPTH_EINVAL;
    const unsigned out_f32 = (flags & TOPTH_OUT_F32) && dtype == TOPTH_BF16 ? kFlagOutF32 : 0u;
    flags &= ~TOPTH_OUT_F32;
    if (pre ? bad_pre_flags(flags, e_tilde, gamma) : (flags & ~(TOPTH_VMC | TOPTH_SDC_NONE)) != 0)
        return TOPTH_EINVAL;
    if ((flags & TOPTH_VMC) && !(flags & TOPTH_SDC_NONE) && !v_mean) return TOPTH_EINVAL;
    if (too_big((long long)B * Hkv * Lmax, d)) return TOPTH_EUNSUPPORTED;
    if (!ws) return TOPTH_EWORKSPACE;
    if (ws_bytes < decode_ws(B, Hq, Hkv, Lmax, d)) return TOPTH_EWORKSPACE;
    DecodeParams p = {};
    p.q = q; p.k = k_cache; p.v = v_cache; p.seq_lens = seq_lens;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Lmax = Lmax; p.d = d; p.dtype = dtype; p.scale = scale;
    p.theta = theta; p.n_rows = n_rows; p.v_mean = v_mean; p.flags = flags | out_f32;
    p.out = out; p.kept_count = kept_count; p.beta = beta; p.vrows_read = vrows_read;
    p.kept_mask = kept_mask; p.ws = ws; p.ws_bytes = ws_bytes;
    if (pre) { p.flags |= kFlagPre; p.e_tilde = e_tilde; p.gamma = gamma; }
    p.min_votes = min_votes; p.augment = augment ? 1 : 0;
    if (dtype == TOPTH_BF16) {
        if (!decode_bf16_supported(d, Hq / Hkv) || (long long)Lmax * d * 2 >= INT_MAX) return TOPTH_EUNSUPPORTED;
        p.v_mean_append = v_mean_append;              // the kernel appends row n - 1 itself
        return map_hip(launch_decode_bf16(p, (hipStream_t)stream));
    }
    if (Lmax > rowwise_max_keys()) return TOPTH_EUNSUPPORTED;
    if (v_mean_append) {                              // fp32: the stand-alone update first, same stream
        const int e = launch_vmean_append(v_cache, nullptr, seq_lens, B, Hkv, Lmax, d, dtype, v_mean_append,
                                          (hipStream_t)stream);
        if (e != 0) return map_hip(e);
    }
    return map_hip(launch_decode_rowwise(p, (uint32_t*)((char*)ws + kWsHeaderBytes),
                                         (hipStream_t)stream));
}

}  // namespace

extern "C" {

int topth_decode(const void* q, const void* k_cache, const void* v_cache, const int* seq_lens,
                 int B, int Hq, int Hkv, int Lmax, int d, int dtype, float scale,
                 const float* theta, int n_rows, const float* v_mean, unsigned flags,
                 void* out, int* kept_count, float* beta, int* vrows_read,
                 unsigned char* kept_mask, void* ws, size_t ws_bytes, void* stream) {
    return decode_common(q, k_cache, v_cache, seq_lens, B, Hq, Hkv, Lmax, d, dtype, scale, theta,
                         n_rows, v_mean, flags, out, kept_count, beta, vrows_read, kept_mask, ws,
                         ws_bytes, stream, false, nullptr, 0.f);
}

int topth_decode_append(const void* q, const void* k_cache, const void* v_cache, const int* seq_lens,
                        int B, int Hq, int Hkv, int Lmax, int d, int dtype, float scale,
                        const float* theta, int n_rows, float* v_mean, unsigned flags,
                        void* out, int* kept_count, float* beta, int* vrows_read,
                        unsigned char* kept_mask, void* ws, size_t ws_bytes, void* stream) {
    if (!v_mean) return TOPTH_EINVAL;                 // the running mean is always updated
    return decode_common(q, k_cache, v_cache, seq_lens, B, Hq, Hkv, Lmax, d, dtype, scale, theta,
                         n_rows, v_mean, flags, out, kept_count, beta, vrows_read, kept_mask, ws,
                         ws_bytes, stream, false, nullptr, 0.f, 1, 0, v_mean);
}

int topth_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int* seq_lens,
                         int B, int Hq, int Hkv, int Lmax, int d, int dtype, float scale,
                         const float* theta, int n_rows, const float* v_mean, unsigned flags,
                         void* out, int* kept_count, float* beta, int* vrows_read,
                         unsigned char* kept_mask, void* stream) {
    // the argument checks of topth_decode, with a workspace that always passes
    // them; the scratch size is checked against the call's own plan below
    if (!q || !k_cache || !v_cache || !seq_lens || !theta || !out) return TOPTH_EINVAL;
    if (bad_dims(B, Hq, Hkv, Lmax, d) || bad_dtype(dtype) || n_rows <= 0) return TOPTH_EINVAL;
    if (!isfinite(scale) || !(scale > 0.0f)) return TOPTH_EINVAL;
    const unsigned out_f32 = (flags & TOPTH_OUT_F32) && dtype == TOPTH_BF16 ? kFlagOutF32 : 0u;
    flags &= ~TOPTH_OUT_F32;
    if ((flags & ~(TOPTH_VMC | TOPTH_SDC_NONE)) != 0) return TOPTH_EINVAL;
    if ((flags & TOPTH_VMC) && !(flags & TOPTH_SDC_NONE) && !v_mean) return TOPTH_EINVAL;
    if (too_big((long long)B * Hkv * Lmax, d)) return TOPTH_EUNSUPPORTED;
    DecodeParams p = {};
    p.q = q; p.k = k_cache; p.v = v_cache; p.seq_lens = seq_lens;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Lmax = Lmax; p.d = d; p.dtype = dtype; p.scale = scale;
    p.theta = theta; p.n_rows = n_rows; p.v_mean = v_mean; p.flags = flags | out_f32;
    p.out = out; p.kept_count = kept_count; p.beta = beta; p.vrows_read = vrows_read;
    p.kept_mask = kept_mask; p.min_votes = 1; p.augment = 0;
    if (dtype == TOPTH_BF16) {
        if (!decode_bf16_supported(d, Hq / Hkv) || (long long)Lmax * d * 2 >= INT_MAX) return TOPTH_EUNSUPPORTED;
        bool fits = false;
        const int e = launch_decode_bf16_noalloc(p, &fits, (hipStream_t)stream);
        if (e != 0) return TOPTH_EHIP;
        return fits ? TOPTH_OK : TOPTH_ESCRATCH;
    }
    if (Lmax > rowwise_max_keys()) return TOPTH_EUNSUPPORTED;
    // the float32 path writes its mask words before it reads them: nothing to prepare
    if (kWsHeaderBytes + decode_rowwise_ws_bytes(B, Hq, Lmax) > noalloc_scratch_bytes()) return TOPTH_ESCRATCH;
    void* ws = nullptr;
    if (noalloc_scratch(&ws) != 0) return TOPTH_EHIP;
    return map_hip(launch_decode_rowwise(p, (uint32_t*)((char*)ws + kWsHeaderBytes), (hipStream_t)stream));
}

int topth_decode_pre(const void* q, const void* k_cache, const void* v_cache, const int* seq_lens,
                     int B, int Hq, int Hkv, int Lmax, int d, int dtype, float scale,
                     const float* theta, const float* e_tilde, int n_rows, const float* v_mean,
                     unsigned flags, float gamma, void* out, int* kept_count, float* beta,
                     int* vrows_read, unsigned char* kept_mask, void* ws, size_t ws_bytes,
                     void* stream) {
    return decode_common(q, k_cache, v_cache, seq_lens, B, Hq, Hkv, Lmax, d, dtype, scale, theta,
                         n_rows, v_mean, flags, out, kept_count, beta, vrows_read, kept_mask, ws,
                         ws_bytes, stream, true, e_tilde, gamma);
}

int topth_vmean(const void* v, const int* seq_lens, int B, int Hkv, int Lmax, int d, int dtype,
                float* v_mean, void* stream) {
    if (!v || !seq_lens || !v_mean) return TOPTH_EINVAL;
    if (bad_dims(B, Hkv, Hkv, Lmax, d) || bad_dtype(dtype)) return TOPTH_EINVAL;
    if (too_big((long long)B * Hkv * Lmax, d)) return TOPTH_EUNSUPPORTED;
    return map_hip(launch_vmean(v, seq_lens, B, Hkv, Lmax, d, dtype, v_mean, (hipStream_t)stream));
}

int topth_vmean_append(const void* v_cache, const int* old_lens, const int* new_lens, int B, int Hkv,
                       int Lmax, int d, int dtype, float* v_mean, void* stream) {
    if (!v_cache || !old_lens || !new_lens || !v_mean) return TOPTH_EINVAL;
    if (bad_dims(B, Hkv, Hkv, Lmax, d) || bad_dtype(dtype)) return TOPTH_EINVAL;
    if (too_big((long long)B * Hkv * Lmax, d)) return TOPTH_EUNSUPPORTED;
    return map_hip(launch_vmean_append(v_cache, old_lens, new_lens, B, Hkv, Lmax, d, dtype, v_mean,
                                       (hipStream_t)stream));
}

int topth_theta_fit(const float* theta, const int* count, const int* ks, int n_k, int Hq, int n_rows,
                    int degree, int log_domain, int min_len_over_k, double* coef, void* stream) {
    if (!theta || !count || !ks || !coef) return TOPTH_EINVAL;
    if (n_k < 1 || n_k > TOPTH_MAX_NK || Hq <= 0 || n_rows <= 0) return TOPTH_EINVAL;
    if (degree < 0 || degree > max_fit_degree() || min_len_over_k < 0) return TOPTH_EINVAL;
    for (int t = 0; t < n_k; ++t)
        if (ks[t] < 1) return TOPTH_EINVAL;
    if ((long long)n_k * Hq > INT_MAX) return TOPTH_EUNSUPPORTED;
    return map_hip(launch_theta_fit(theta, count, ks, n_k, Hq, n_rows, degree, log_domain != 0, min_len_over_k,
                                    coef, (hipStream_t)stream));
}

int topth_theta_eval(const double* coef, const int* ks, int n_k, int Hq, int degree, int log_domain,
                     int n_out, float* theta_out, void* stream) {
    if (!coef || !ks || !theta_out) return TOPTH_EINVAL;
    if (n_k < 1 || n_k > TOPTH_MAX_NK || Hq <= 0 || n_out <= 0) return TOPTH_EINVAL;
    if (degree < 0 || degree > max_fit_degree()) return TOPTH_EINVAL;
    for (int t = 0; t < n_k; ++t)
        if (ks[t] < 1) return TOPTH_EINVAL;
    if ((long long)n_k * Hq > 65535) return TOPTH_EUNSUPPORTED;     // one grid row per (t, h)
    return map_hip(launch_theta_eval(coef, ks, n_k, Hq, degree, log_domain != 0, n_out, theta_out,
                                     (hipStream_t)stream));
}

int topth_decode_gqa(const void* q, const void* k_cache, const void* v_cache, const int* seq_lens,
                     int B, int Hq, int Hkv, int Lmax, int d, int dtype, float scale,
                     const float* theta, int n_rows, const float* v_mean, unsigned flags,
                     int min_votes, int augment, void* out, int* kept_count, float* beta,
                     int* vrows_read, unsigned char* kept_mask, void* ws, size_t ws_bytes,
                     void* stream) {
    if (Hkv <= 0 || Hq <= 0 || (Hq % Hkv) != 0) return TOPTH_EINVAL;
    if (min_votes < 1 || min_votes > Hq / Hkv || (augment != 0 && augment != 1)) return TOPTH_EINVAL;
    return decode_common(q, k_cache, v_cache, seq_lens, B, Hq, Hkv, Lmax, d, dtype, scale, theta,
                         n_rows, v_mean, flags, out, kept_count, beta, vrows_read, kept_mask, ws,
                         ws_bytes, stream, false, nullptr, 0.f, min_votes, augment);
}

}  // extern "C"
