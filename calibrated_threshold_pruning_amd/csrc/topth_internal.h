// Internal declarations and device helpers of libtopth (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace topth {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;

// Workspace: a header (status word at byte 0, spin limit at byte 4, the rest
// reserved), then the decode exchange slots.  An empty slot holds kWsSlotEmpty in every 32-bit
// word: a NaN payload that float arithmetic never produces (it returns the
// default NaN 0x7FC00000) and no count or length reaches as an integer.
constexpr size_t kWsHeaderBytes = 65536;
constexpr uint32_t kWsSlotEmpty = 0x7FC0DEADu;
constexpr int kStatusSpinTimeout = 1;
// static device scratch of the no-allocation decode entry point, per GPU
constexpr size_t kNoallocScratchBytes = (size_t)80 << 20;

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// round-to-nearest-even float -> bfloat16 bits (NaN stays NaN)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float* p) { return *p; }
    static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Elem<uint16_t> {   // bfloat16 stored as raw bits
    static __device__ __forceinline__ float load(const uint16_t* p) { return bf16_bits_to_f32(*p); }
    static __device__ __forceinline__ void store(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }
};

// order-preserving map float -> uint32 (larger float <-> larger key)
__device__ __forceinline__ uint32_t float_to_ordered(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ordered_to_float(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

// ------------------------------------------------------------ wave reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// threshold in the log2 domain: keep x >= T  <=>  s = exp2(x - lse2) >= theta.
// theta <= 0 or -inf keeps every valid element; invalid elements carry x = -inf
// and never pass because T is clamped to -FLT_MAX.
__device__ __forceinline__ float log2_threshold(float theta, float lse2) {
    if (!(theta > 0.0f)) return -3.402823466e38f;
    return fmaxf(__log2f(theta) + lse2, -3.402823466e38f);
}

// pre-softmax threshold in the log2 domain: keep x = a * log2(e) >= T  <=>  a >= theta;
// theta = -inf keeps every valid element (invalid ones carry x = -inf)
__device__ __forceinline__ float pre_log2_threshold(float theta) {
    return fmaxf(theta * kLog2e, -3.402823466e38f);
}

// Flag bits of the kernels (the public TOPTH_* values, plus kFlagPre for the
// pre-softmax calls).  kFlagExpth / kFlagOffline select the estimate of the
// discarded softmax mass E~; neither (and not kFlagNone) means exact E.
constexpr unsigned kFlagVmc = 0x1u, kFlagNone = 0x2u, kFlagExpth = 0x4u, kFlagOffline = 0x8u;
constexpr unsigned kFlagOutF32 = 0x10u;   // bfloat16 inputs: out is float32
constexpr unsigned kFlagPre = 0x100u;

// Scale f and beta of a row from its kept post-softmax mass S = R / (R + E),
// written in the frame where the full denominator R + E is 1 (Eq. 4):
// out = f * sum_kept s_j V_j + beta * mu with f = 1 / (S + E~ / (R + E)) and
// beta = 1 - f * S.  etn = E~ / (R + E): 1 - S for exact SDC (f = 1), 0 for
// no compensation (f = 1 / S, beta = 0).  A zero denominator gives f = beta = 0.
__device__ __forceinline__ void sdc_scale(unsigned flags, float S, int kept, float etn, float& f,
                                          float& beta) {
    if (!(flags & kFlagNone) && !(flags & (kFlagExpth | kFlagOffline))) {   // exact
        f = 1.f;
        beta = 1.f - S;
        return;
    }
    const float den = (flags & kFlagNone) ? S : S + etn;
    if (!(den > 0.f) || ((flags & kFlagNone) && kept == 0)) { f = 0.f; beta = 0.f; return; }
    f = 1.f / den;
    beta = (flags & kFlagNone) ? 0.f : 1.f - f * S;
}

// ------------------------------------------------------------------ launchers
struct DecodeParams {
    const void* q; const void* k; const void* v; const int* seq_lens;
    int B, Hq, Hkv, Lmax, d, dtype; float scale;
    const float* theta; int n_rows; const float* v_mean; unsigned flags;
    void* out; int* kept_count; float* beta; int* vrows_read; unsigned char* kept_mask;
    void* ws; size_t ws_bytes;
    const float* e_tilde; float gamma;    // pre-softmax calls only
    int min_votes; int augment;           // GQA selection variants (0, 0: plain per-head selection)
    float* v_mean_append;                 // non-NULL: append row n - 1 to this running mean, then use it
};
struct PrefillParams {
    const void* q; const void* k; const void* v;
    int B, Hq, Hkv, L, d, dtype; float scale;
    const float* theta; int n_rows; unsigned flags;
    void* out; int* kept_count; float* beta; unsigned char* kept_mask;
    void* ws; size_t ws_bytes;
    const float* e_tilde; float gamma;    // pre-softmax calls only
};
struct CalibParams {
    const void* q; const void* k;
    int S, Hq, Hkv, Lq, Lk, d, dtype; float scale; int q_pos0;
    int ks[8]; int n_k;
    double* sum; double* sumsq; int* count; int n_rows;
    void* ws; size_t ws_bytes;
    bool pre; double* esum;               // pre-softmax samples; E~ sums or NULL
    const int* mkc_ks;                    // multi-k calibration: host [n_k] target k (n_k <= 64)
};

// Each launcher validates nothing (the ABI layer did) and returns a hipError_t.
size_t decode_ws_bytes(int B, int Hq, int Hkv, int Lmax, int d);
int launch_decode(const DecodeParams& p, hipStream_t s);
size_t prefill_ws_bytes(int B, int Hq, int Hkv, int L, int d);
int launch_prefill(const PrefillParams& p, hipStream_t s);
size_t calib_ws_bytes(int S, int Hq, int Lq, int Lk, int d, int n_k);
int launch_calibrate(const CalibParams& p, hipStream_t s);
int launch_finalize(const double* sum, const double* sumsq, const int* count, const int* ks,
                    int n_k, int Hq, int n_rows, float alpha, float* theta, hipStream_t s);
int launch_finalize_etilde(const double* esum, const int* count, const int* ks, int n_k, int Hq,
                           int n_rows, float* e_tilde, hipStream_t s);
int launch_vmean(const void* v, const int* seq_lens, int B, int Hkv, int Lmax, int d, int dtype,
                 float* v_mean, hipStream_t s);
int launch_fill_u32(void* p, size_t bytes, uint32_t value, hipStream_t s);
int launch_ws_prepare(void* ws, size_t header_bytes, size_t end_bytes, hipStream_t s);

}  // namespace topth
