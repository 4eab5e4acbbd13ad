// Top-theta decode for bfloat16 KV caches on gfx950.
//
// One generative-decoding step ("Top-Theta Attention: Sparsifying Transformers
// by Compensated Thresholding", Sec. 2.2 decode phase): every query head scores
// all n cached keys, keeps the post-softmax elements s_j >= theta (Sec. 3),
// weights them by s_j itself (exact SDC, Sec. 3.2.1 Eq. 4), adds beta * mu
// (VMC, Sec. 3.2.2 Eq. 5-7), and -- the point of the method in decoding -- only
// the V rows that some head of the GQA group keeps are read (Sec. 4.6).
//
// Kernel shape (persistent, cooperative launch so every workgroup is resident):
//   work item = (group = (b, kv head), chunk of keys); 4 waves per workgroup.
//   Phase 1  each wave streams its keys' K rows straight from HBM in the MFMA
//            B-operand layout and forms the g scores per key with
//            v_mfma_f32_16x16x32_bf16 (query heads in the A operand, several
//            key tiles packed into the 16 rows when g < 16).  Scores stay in
//            registers; the wave and the workgroup reduce per-head (max, sum
//            of exp2) and publish them.
//   Exchange the chunks of a group meet at a counter in the workspace; every
//            chunk then combines all partials in the same order, so all see the
//            same row log-sum-exp.
//   Phase 2  compare x >= log2(theta) + lse2 per (key, head); OR over the
//            group's heads; ballot + popcount compaction of the kept keys into
//            a per-wave LDS list; gather only those V rows with 16 lanes x
//            16 bytes per 256-byte row; accumulate s * V per head in float32.
//   Combine  the last chunk of a group to finish sums the chunk partials in a
//            fixed order and applies beta * mu.
// Reductions never use float atomics, so results are run-to-run identical.
#include "topth_internal.h"

#include <math.h>

namespace topth {

struct DecodeKArgs {
    const uint16_t* q; const uint16_t* k; const uint16_t* v; const int* seq_lens;
    const float* theta; const float* v_mean;
    uint16_t* out; int* kept_count; float* beta; int* vrows_read; unsigned char* kept_mask;
    int* status; int* counters;
    float2* part_ml; float* part_out; float* part_mass; int* part_cnt; int* part_union;
    int B, Hq, Hkv, Lmax, n_rows, chunks, items;
    float xscale;
    unsigned flags;
    unsigned spin_limit;
};

template <int D, int G, int NT>
struct DecodeCfg {
    static constexpr int P = (G <= 4) ? 4 : (G == 8 ? 2 : 1);  // key tiles packed per MFMA
    static constexpr int GP = 16 / P;          // A-operand rows per key tile (heads, padded)
    static constexpr int BPT = 4 / P;          // 16-lane blocks per key tile
    static constexpr int KT = 16 * P;          // keys per wave tile
    static constexpr int STEPS = D * P / 32;   // MFMA steps over the head dimension
    static constexpr int WAVES = 4;
    static constexpr int THREADS = WAVES * 64;
    static constexpr int KEYS_PER_WG = WAVES * NT * KT;
    static constexpr int GW = G < 4 ? 4 : G;   // heads per LDS weight row (padded to 4)
    static constexpr int DPL = D / 16;         // V dims per lane in the gather
    static_assert(STEPS >= 1, "head dimension too small");
};

template <int DPL> struct VVec;
template <> struct VVec<8> { typedef u32x4 T; };
template <> struct VVec<4> { typedef uint2 T; };

__device__ __forceinline__ void unpack_bf16(const u32x4& u, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(u[i] << 16);
        f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void unpack_bf16(const uint2& u, float* f) {
    f[0] = __uint_as_float(u.x << 16); f[1] = __uint_as_float(u.x & 0xffff0000u);
    f[2] = __uint_as_float(u.y << 16); f[3] = __uint_as_float(u.y & 0xffff0000u);
}

template <int D, int G, int NT>
__global__ __launch_bounds__(256) void decode_bf16_kernel(DecodeKArgs a) {
    using C = DecodeCfg<D, G, NT>;
    __shared__ float s_m[C::WAVES][G], s_l[C::WAVES][G];
    __shared__ float s_T[G], s_lse[G];
    __shared__ __attribute__((aligned(16))) float s_w[C::WAVES][C::KT][C::GW];
    __shared__ int s_list[C::WAVES][C::KT];
    __shared__ float s_red[C::WAVES][G][D];
    __shared__ float s_cm[C::WAVES][G];
    __shared__ int s_cc[C::WAVES][G];
    __shared__ int s_un[C::WAVES];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int blk = lane >> 4;                 // 16-lane block of the MFMA operands
    const int cc = blk % C::BPT;               // block inside its key tile
    const int tt = blk / C::BPT;               // key tile of this lane
    const int mykey = (lane & 15) + 16 * tt;   // key of this lane inside a wave tile
    const int hb = 4 * cc;                     // first head of this lane's C registers
    const float NEG_INF = -INFINITY;

    for (int item = blockIdx.x; item < a.items; item += gridDim.x) {
        const int group = item / a.chunks, chunk = item % a.chunks;
        const int b = group / a.Hkv, kv = group % a.Hkv;
        const int n = min(max(a.seq_lens[b], 1), a.Lmax);   // lengths outside [1, Lmax] are clamped
        const int wbase = chunk * C::KEYS_PER_WG + wave * NT * C::KT;

        // ---- query fragments: A[i][k], row i = lane % 16 (head of key tile i / GP)
        bf16x8 qa[C::STEPS];
        {
            const int i = lane & 15;
            const int hi = i % C::GP;
            const bool valid = (i / C::GP == tt) && (hi < G);
            const uint16_t* qrow = a.q + ((size_t)b * a.Hq + (size_t)kv * G + (valid ? hi : 0)) * D;
#pragma unroll
            for (int s = 0; s < C::STEPS; ++s) {
                const u32x4 raw = *(const u32x4*)(qrow + (s * C::BPT + cc) * 8);
                const u32x4 z = {0u, 0u, 0u, 0u};
                qa[s] = __builtin_bit_cast(bf16x8, valid ? raw : z);
            }
        }

        // ---- phase 1: scores of this wave's keys, kept in registers
        const uint16_t* kg = a.k + (size_t)group * a.Lmax * D;
        f32x4 sc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int key0 = wbase + t * C::KT;
            sc[t] = f32x4{NEG_INF, NEG_INF, NEG_INF, NEG_INF};
            if (key0 < n) {
                const int key = key0 + mykey;
                const int keyc = key < a.Lmax ? key : a.Lmax - 1;
                const u32x4* kp = (const u32x4*)(kg + (size_t)keyc * D) + cc;
                u32x4 kb[C::STEPS];
#pragma unroll
                for (int s = 0; s < C::STEPS; ++s) kb[s] = kp[s * C::BPT];
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < C::STEPS; ++s)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        qa[s], __builtin_bit_cast(bf16x8, kb[s]), acc, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool ok = (key < n) && (hb + r < G);
                    sc[t][r] = ok ? acc[r] * a.xscale : NEG_INF;
                }
            }
        }

        // per-head max and sum of exp2 over this wave, then the workgroup
        float mr[4], lr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float m = NEG_INF;
#pragma unroll
            for (int t = 0; t < NT; ++t) m = fmaxf(m, sc[t][r]);
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
            if (C::BPT == 1) { m = fmaxf(m, __shfl_xor(m, 16)); m = fmaxf(m, __shfl_xor(m, 32)); }
            if (C::BPT == 2) m = fmaxf(m, __shfl_xor(m, 32));
            float l = 0.f;
            if (m != NEG_INF) {
#pragma unroll
                for (int t = 0; t < NT; ++t) l += exp2f(sc[t][r] - m);
            }
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) l += __shfl_xor(l, o);
            if (C::BPT == 1) { l += __shfl_xor(l, 16); l += __shfl_xor(l, 32); }
            if (C::BPT == 2) l += __shfl_xor(l, 32);
            mr[r] = m; lr[r] = l;
        }
        if ((lane & 15) == 0 && tt == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (hb + r < G) { s_m[wave][hb + r] = mr[r]; s_l[wave][hb + r] = lr[r]; }
        }
        __syncthreads();
        if (tid < G) {
            float M = NEG_INF;
            for (int w = 0; w < C::WAVES; ++w) M = fmaxf(M, s_m[w][tid]);
            float L = 0.f;
            if (M != NEG_INF)
                for (int w = 0; w < C::WAVES; ++w) L += s_l[w][tid] * exp2f(s_m[w][tid] - M);
            a.part_ml[((size_t)group * a.chunks + chunk) * G + tid] = make_float2(M, L);
        }

        // ---- exchange: wait until every chunk of the group has published
        __threadfence();
        __syncthreads();
        if (tid == 0) {
            int* ctr = a.counters + 2 * group;
            atomicAdd(ctr, 1);
            unsigned spins = 0;
            while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < a.chunks) {
                __builtin_amdgcn_s_sleep(2);
                if (++spins > a.spin_limit) { atomicOr(a.status, kStatusSpinTimeout); break; }
            }
            __threadfence();
        }
        __syncthreads();
        if (tid < G) {
            const float2* pm = a.part_ml + (size_t)group * a.chunks * G + tid;
            float M = NEG_INF;
            for (int c = 0; c < a.chunks; ++c) M = fmaxf(M, pm[(size_t)c * G].x);
            float L = 0.f;
            for (int c = 0; c < a.chunks; ++c) {
                const float2 v = pm[(size_t)c * G];
                if (v.y > 0.f) L += v.y * exp2f(v.x - M);
            }
            const float lse2 = M + __log2f(L);
            const int h = kv * G + tid;
            const float th = a.theta[(size_t)h * a.n_rows + min(n - 1, a.n_rows - 1)];
            s_T[tid] = log2_threshold(th, lse2);
            s_lse[tid] = lse2;
        }
        __syncthreads();

        // ---- phase 2: threshold, compaction, sparse V gather
        float Tr[4], Lr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool hv = hb + r < G;
            Tr[r] = hv ? s_T[hb + r] : INFINITY;
            Lr[r] = hv ? s_lse[hb + r] : 0.f;
        }
        float kmass[4] = {0.f, 0.f, 0.f, 0.f};
        int kcnt[4] = {0, 0, 0, 0};
        int ucount = 0;
        float acc[G][C::DPL];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int i = 0; i < C::DPL; ++i) acc[h][i] = 0.f;

        const unsigned long long keylanes =
            C::BPT == 1 ? ~0ull : (C::BPT == 2 ? 0x0000ffff0000ffffull : 0xffffull);
        const uint16_t* vg = a.v + (size_t)group * a.Lmax * D;

#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int key0 = wbase + t * C::KT;
            if (key0 < n) {
                float w[4];
                int any = 0;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool kp = sc[t][r] >= Tr[r];
                    w[r] = kp ? exp2f(sc[t][r] - Lr[r]) : 0.f;
                    kcnt[r] += kp ? 1 : 0;
                    kmass[r] += w[r];
                    any |= kp ? 1 : 0;
                    if (a.kept_mask && hb + r < G && key0 + mykey < a.Lmax)
                        a.kept_mask[((size_t)b * a.Hq + (size_t)kv * G + hb + r) * a.Lmax + key0 + mykey] =
                            kp ? 1 : 0;
                }
                if (C::BPT >= 2) any |= __shfl_xor(any, 16);
                if (C::BPT == 4) any |= __shfl_xor(any, 32);
                const unsigned long long bal = __ballot(any) & keylanes;
                const int cnt = __popcll(bal);
                if (cnt) {
                    if (hb < C::GW) {
                        float4 wv = make_float4(w[0], w[1], w[2], w[3]);
                        *(float4*)&s_w[wave][mykey][hb] = wv;
                    }
                    if (any && cc == 0) {
                        const unsigned long long below = (lane == 0) ? 0ull : (bal & (~0ull >> (64 - lane)));
                        s_list[wave][__popcll(below)] = mykey;
                    }
                    ucount += cnt;
                    const uint16_t* vt = vg + (size_t)key0 * D + (lane & 15) * C::DPL;
                    for (int e0 = 0; e0 < cnt; e0 += 4) {
                        const int e = e0 + blk;
                        const bool act = e < cnt;
                        const int kp = act ? s_list[wave][e] : 0;
                        typename VVec<C::DPL>::T raw = *(const typename VVec<C::DPL>::T*)(vt + (size_t)kp * D);
                        float vf[C::DPL];
                        unpack_bf16(raw, vf);
                        float wh[C::GW];
#pragma unroll
                        for (int q4 = 0; q4 < C::GW; q4 += 4) {
                            const float4 x = *(const float4*)&s_w[wave][kp][q4];
                            wh[q4] = x.x; wh[q4 + 1] = x.y; wh[q4 + 2] = x.z; wh[q4 + 3] = x.w;
                        }
#pragma unroll
                        for (int h = 0; h < G; ++h) {
                            const float ww = act ? wh[h] : 0.f;
#pragma unroll
                            for (int i = 0; i < C::DPL; ++i) acc[h][i] = fmaf(ww, vf[i], acc[h][i]);
                        }
                    }
                }
            }
        }

        // ---- partial results of this workgroup
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int i = 0; i < C::DPL; ++i) {
                float x = acc[h][i];
                x += __shfl_xor(x, 16);
                x += __shfl_xor(x, 32);
                acc[h][i] = x;
            }
        if (lane < 16) {
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int i = 0; i < C::DPL; ++i) s_red[wave][h][lane * C::DPL + i] = acc[h][i];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float m = kmass[r];
            int c = kcnt[r];
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) { m += __shfl_xor(m, o); c += __shfl_xor(c, o); }
            if (C::BPT == 1) {
                m += __shfl_xor(m, 16); c += __shfl_xor(c, 16);
                m += __shfl_xor(m, 32); c += __shfl_xor(c, 32);
            }
            if (C::BPT == 2) { m += __shfl_xor(m, 32); c += __shfl_xor(c, 32); }
            kmass[r] = m; kcnt[r] = c;
        }
        if ((lane & 15) == 0 && tt == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (hb + r < G) { s_cm[wave][hb + r] = kmass[r]; s_cc[wave][hb + r] = kcnt[r]; }
        }
        if (lane == 0) s_un[wave] = ucount;
        __syncthreads();
        const size_t pbase = (size_t)group * a.chunks + chunk;
        for (int idx = tid; idx < G * D; idx += C::THREADS) {
            float x = 0.f;
#pragma unroll
            for (int w = 0; w < C::WAVES; ++w) x += (&s_red[w][0][0])[idx];
            a.part_out[pbase * G * D + idx] = x;
        }
        if (tid < G) {
            float m = 0.f; int c = 0;
            for (int w = 0; w < C::WAVES; ++w) { m += s_cm[w][tid]; c += s_cc[w][tid]; }
            a.part_mass[pbase * G + tid] = m;
            a.part_cnt[pbase * G + tid] = c;
        }
        if (tid == 0) {
            int u = 0;
            for (int w = 0; w < C::WAVES; ++w) u += s_un[w];
            a.part_union[pbase] = u;
        }

        // ---- the last chunk of the group to finish combines
        __threadfence();
        __syncthreads();
        if (tid == 0) {
            const int old = atomicAdd(a.counters + 2 * group + 1, 1);
            s_last = (old == a.chunks - 1);
            if (s_last) __threadfence();
        }
        __syncthreads();
        if (s_last) {
            const bool renorm = (a.flags & 2u) != 0;
            const bool vmc = (a.flags & 1u) != 0 && !renorm;
            const size_t g0 = (size_t)group * a.chunks;
            if (tid < G) {
                float m = 0.f; int c = 0;
                for (int ch = 0; ch < a.chunks; ++ch) {
                    m += a.part_mass[(g0 + ch) * G + tid];
                    c += a.part_cnt[(g0 + ch) * G + tid];
                }
                s_cm[0][tid] = m;
                s_cc[0][tid] = c;
                const size_t o = (size_t)b * a.Hq + (size_t)kv * G + tid;
                if (a.kept_count) a.kept_count[o] = c;
                if (a.beta) a.beta[o] = renorm ? 0.f : 1.f - m;
            }
            if (tid == 0 && a.vrows_read) {
                int u = 0;
                for (int ch = 0; ch < a.chunks; ++ch) u += a.part_union[g0 + ch];
                a.vrows_read[group] = u;
            }
            __syncthreads();
            for (int idx = tid; idx < G * D; idx += C::THREADS) {
                const int h = idx / D, dd = idx % D;
                float x = 0.f;
                for (int ch = 0; ch < a.chunks; ++ch) x += a.part_out[((g0 + ch) * G) * D + idx];
                const float mass = s_cm[0][h];
                if (renorm) x = (s_cc[0][h] > 0) ? x / mass : 0.f;
                if (vmc) x = fmaf(1.f - mass, a.v_mean[(size_t)group * D + dd], x);
                a.out[((size_t)b * a.Hq + (size_t)kv * G + h) * D + dd] = f32_to_bf16_bits(x);
            }
            if (tid == 0) {
                __hip_atomic_store(a.counters + 2 * group, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(a.counters + 2 * group + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ host side
namespace {

typedef void (*DecodeKernelFn)(DecodeKArgs);

struct Variant {
    DecodeKernelFn fn;
    int keys_per_wg;
    int nt;
};

template <int D, int G>
Variant variant_for(int nt_index) {
    switch (nt_index) {
        case 0: return {decode_bf16_kernel<D, G, 4>, DecodeCfg<D, G, 4>::KEYS_PER_WG, 4};
        case 1: return {decode_bf16_kernel<D, G, 8>, DecodeCfg<D, G, 8>::KEYS_PER_WG, 8};
        case 2: return {decode_bf16_kernel<D, G, 16>, DecodeCfg<D, G, 16>::KEYS_PER_WG, 16};
        default:
            if (G == 16) return {decode_bf16_kernel<D, G, 16>, DecodeCfg<D, G, 16>::KEYS_PER_WG, 16};
            return {decode_bf16_kernel<D, G, (G == 16 ? 16 : 32)>,
                    DecodeCfg<D, G, (G == 16 ? 16 : 32)>::KEYS_PER_WG, (G == 16 ? 16 : 32)};
    }
}

template <int D>
Variant pick_variant(int G, int nt_index) {
    switch (G) {
        case 1: return variant_for<D, 1>(nt_index);
        case 2: return variant_for<D, 2>(nt_index);
        case 4: return variant_for<D, 4>(nt_index);
        case 8: return variant_for<D, 8>(nt_index);
        default: return variant_for<D, 16>(nt_index);
    }
}

Variant pick(int d, int G, int nt_index) {
    return d == 64 ? pick_variant<64>(G, nt_index) : pick_variant<128>(G, nt_index);
}

int keys_per_wg_min(int G) {
    const int P = (G <= 4) ? 4 : (G == 8 ? 2 : 1);
    return 4 * 4 * 16 * P;
}

int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return cus;
}

}  // namespace

bool decode_bf16_supported(int d, int G) {
    return (d == 64 || d == 128) && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
}

size_t decode_ws_bytes(int B, int Hq, int Hkv, int Lmax, int d) {
    const int G = Hq / Hkv;
    const size_t groups = (size_t)B * Hkv;
    const size_t chunks = (size_t)((Lmax + keys_per_wg_min(G) - 1) / keys_per_wg_min(G));
    const size_t pc = groups * chunks;
    size_t bytes = kWsHeaderBytes;
    bytes += pc * G * sizeof(float2);
    bytes += pc * G * d * sizeof(float);
    bytes += pc * G * sizeof(float);
    bytes += pc * G * sizeof(int);
    bytes += pc * sizeof(int);
    return bytes + 256;
}

// Spin limit of the in-kernel exchange; a host test may lower it.
static unsigned g_spin_limit = 1u << 22;
void decode_set_spin_limit(unsigned v) { g_spin_limit = v; }

int launch_decode_bf16(const DecodeParams& p, hipStream_t stream) {
    const int G = p.Hq / p.Hkv;
    const int groups = p.B * p.Hkv;
    const int cus = device_cus();
    if (cus <= 0) return hipErrorNoDevice;

    // choose the smallest register footprint whose work fits in one resident round
    Variant v{};
    int chunks = 0, capacity = 0;
    for (int ni = 0; ni < 4; ++ni) {
        Variant cand = pick(p.d, G, ni);
        int per_cu = 0;
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)cand.fn, 256, 0);
        if (e != hipSuccess) return e;
        const int cap = per_cu * cus;
        const int ch = (p.Lmax + cand.keys_per_wg - 1) / cand.keys_per_wg;
        v = cand; chunks = ch; capacity = cap;
        if ((long long)ch * groups <= cap) break;
    }
    if (chunks > capacity || capacity <= 0) return hipErrorInvalidConfiguration;
    const int items = chunks * groups;
    const int grid = std::min(items, (capacity / chunks) * chunks);

    // workspace carve-up (the header holds status and counters)
    char* ws = (char*)p.ws;
    DecodeKArgs a = {};
    a.q = (const uint16_t*)p.q; a.k = (const uint16_t*)p.k; a.v = (const uint16_t*)p.v;
    a.seq_lens = p.seq_lens; a.theta = p.theta; a.v_mean = p.v_mean;
    a.out = (uint16_t*)p.out; a.kept_count = p.kept_count; a.beta = p.beta; a.vrows_read = p.vrows_read;
    a.kept_mask = p.kept_mask;
    a.status = (int*)ws;
    a.counters = (int*)ws + kWsCounterOffsetInts;
    size_t off = kWsHeaderBytes;
    const size_t pc = (size_t)items;
    a.part_ml = (float2*)(ws + off); off += pc * G * sizeof(float2);
    a.part_out = (float*)(ws + off); off += pc * G * p.d * sizeof(float);
    a.part_mass = (float*)(ws + off); off += pc * G * sizeof(float);
    a.part_cnt = (int*)(ws + off); off += pc * G * sizeof(int);
    a.part_union = (int*)(ws + off); off += pc * sizeof(int);
    if (off > p.ws_bytes) return hipErrorInvalidValue;
    a.B = p.B; a.Hq = p.Hq; a.Hkv = p.Hkv; a.Lmax = p.Lmax; a.n_rows = p.n_rows;
    a.chunks = chunks; a.items = items;
    a.xscale = p.scale * kLog2e;
    a.flags = p.flags;
    a.spin_limit = g_spin_limit;

    void* args[] = {&a};
    return hipLaunchCooperativeKernel((const void*)v.fn, dim3(grid), dim3(256), args, 0, stream);
}

}  // namespace topth
