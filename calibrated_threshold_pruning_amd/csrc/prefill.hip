// Top-theta prefill for bfloat16 inputs on gfx950.
//
// Causal attention of every query row p over keys 0..p ("Top-Theta Attention:
// Sparsifying Transformers by Compensated Thresholding", Eq. 1-3 with the
// 1/sqrt(d) scale and causal mask of Sec. 2.2), keeping the post-softmax
// elements s >= theta[h][p] (Sec. 3), weighting them by s itself (exact SDC,
// Sec. 3.2.1 Eq. 4) and optionally adding beta * mu_p (VMC, Sec. 3.2.2).
//
// Post-softmax thresholding needs the exact row log-sum-exp before the first
// compare, so every query tile sweeps its causal key range twice:
//   sweep A  S^T = K Q^T on MFMA; a lane-local sum of exp2 against a lazily
//            raised reference maximum; the four lanes of a row combine into
//            the row LSE at the end.
//   sweep B  S^T again; compare x >= log2(theta) + lse2; P = exp2(x - lse2)
//            for kept elements (0 otherwise) is taken straight from the
//            accumulator registers as the B operand of O^T += V^T P^T, split
//            into a bf16 high part and a bf16 remainder (two MFMAs).
// Workgroup: one KV head's query tile, 4 waves, each wave one query head and
// 32 rows; K tiles of 64 keys are staged by buffer_load...lds into a swizzled,
// double-buffered LDS tile shared by the waves; V tiles are staged as they
// are and read transposed (bf16), or come as float16 V^T image tiles.
//
// Pre-softmax form (PRE): the compare a >= theta needs no row statistics, so
// sweep A is skipped and sweep B alone keeps an online softmax: a row-uniform
// reference maximum, raised lazily (only when a tile's maximum exceeds it by
// more than 2^8 in exp2 units, which bounds every weight by 256), with the
// output accumulators, the full sum and the kept sum R rescaled when it moves.
// The epilogue divides by R + E~ for the chosen estimate of the discarded mass
// (Sec. 3.2.1: exact, exp-threshold, offline-calibrated, or none).
//
// P V in float16: when the caller's workspace has room, a pre-pass copies V to
// float16 V^T tiles laid out as the kernel's LDS tile, so that every V^T
// fragment is one plain 16-byte LDS read (the conversion is exact for
// bfloat16 values of magnitude in [2^-14, 16] and zero; smaller ones land on
// the float16 subnormal grid, off by at most 2^-25, which moves an output by
// at most 2^-25 since the weights sum to at most 1; the bound of 16 is
// checked), and the P V product takes one f16 MFMA per block with P rounded
// to float16 instead of the two bf16 MFMAs of the high/low split.  P enters
// scaled by 2^7 (folded into the exp2 offset of the row, undone in the
// epilogue): a weight is at most 2^8 * 2^7 in float16, and only weights below
// 2^-21 fall into the float16 subnormals, whose absolute rounding error is at
// most 2^-25 * 2^-7.  Per output: 2^-11 * 16 from the relative rounding of the
// normal weights (they sum to at most 1 after normalisation) plus at most
// L * 2^-32 * 16 from the subnormal ones, under 8.1e-3 for L <= 2^16.  A V
// element beyond 16 (or not finite) sets a flag.  Both kernels (F16 and not)
// are launched; each reads the flag first and only the one that matches it
// does the work (the other grid exits at once), so neither carries the
// other's registers.
#include "topth_internal.h"

#include <math.h>

#include <type_traits>

namespace topth {

struct PrefillKArgs {
    const uint16_t* q; const uint16_t* k; const uint16_t* v;
    const float* theta; const float* mu;
    uint16_t* out; int* kept_count; float* beta; unsigned char* kept_mask;
    int B, Hq, Hkv, L, n_rows;
    float xscale;
    unsigned flags;
    float scale;                 // score scale (pre-softmax thresholds are in score units)
    const float* e_tilde;        // offline estimate of E~ [Hq][n_rows] or NULL
    float gamma;                 // exp-threshold estimate
    const uint16_t* v16;         // float16 copy of V, or NULL (bf16 high/low split for P V)
    const unsigned* vflag;       // nonzero: some V element is beyond the float16 bound
};

template <int D, int G>
struct PrefillCfg {
    static constexpr int HPW = G < 4 ? G : 4;       // query heads per workgroup
    static constexpr int RBW = 4 / HPW;             // 32-row blocks per workgroup
    static constexpr int BMT = 32 * RBW;            // query rows per workgroup
    static constexpr int BN = 64;                   // keys per tile
    static constexpr int KSTEPS = D / 32;           // MFMA steps over the head dimension
    static constexpr int DB = D / 16;               // 16-wide dimension blocks of the output
    static constexpr int CPR = D / 8;               // 16-byte chunks per K row
    static constexpr int RPI = 64 / CPR;            // K rows per 1 KiB load instruction
    static constexpr int KTILE = BN * D * 2;        // bytes of one K tile (and of one V^T image tile)
    static constexpr int VROW = BN * 2;             // bytes of one dimension row of a V^T image tile
    static constexpr int NLD = KTILE / 1024 / 4;    // load instructions per wave per K tile
};

__device__ __forceinline__ float pf_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ void pf_wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// wait until at most N vector memory loads of this wave are outstanding (N < 16)
template <int N>
__device__ __forceinline__ void pf_wait_vmem_n() {
    static_assert(N >= 0 && N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Scheduling hint for one region: REPS times, NDS LDS reads then NMFMA MFMAs,
// which puts the reads of the next operand fragments ahead of the MFMAs of the
// current ones instead of right before them.
template <int REPS, int NDS, int NMFMA>
__device__ __forceinline__ void pf_ds_mfma_pipeline() {
#pragma unroll
    for (int i = 0; i < REPS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, NDS, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, NMFMA, 0);
    }
}

typedef __bf16 pf_bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 pf_f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 pf_f16x8 __attribute__((ext_vector_type(8)));
typedef short pf_i16x4 __attribute__((ext_vector_type(4)));
typedef float pf_f32x2 __attribute__((ext_vector_type(2)));

// two floats to packed bfloat16, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
    const pf_f32x2 v = {lo, hi};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, pf_bf16x2));
}
// two floats to packed float16, round to nearest even
__device__ __forceinline__ unsigned pack_f16x2(float lo, float hi) {
    const pf_f32x2 v = {lo, hi};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, pf_f16x2));
}
// P = hi + lo with both parts in bfloat16: the P V product is taken as two bf16
// MFMAs, which keeps about 16 significant bits of every weight
__device__ __forceinline__ void split_bf16x2(float a, float b, unsigned& hi, unsigned& lo) {
    hi = pack_bf16x2(a, b);
    lo = pack_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// MASS: the kept mass of each row is summed (VMC, SDC_NONE, the beta output
// and every pre-softmax estimate need it); without it sweep B skips that sum.
template <int D, int G, bool MASK, bool PRE, bool F16, bool MASS>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(PrefillKArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)   // the host pass only needs the launch stub
    using C = PrefillCfg<D, G>;
    constexpr int PSC = F16 ? 7 : 0;                       // log2 of the P scale of the float16 P V form
    // four tile slots: sweep B double-buffers K in slots 0-1 and V in slots
    // 2-3; sweep A, which reads no V, rotates K through all four
    __shared__ __attribute__((aligned(16))) unsigned char s_kv[4][C::KTILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, lq = lane >> 4;
    const float NEG_INF = -INFINITY;

    // longest query tiles first: they have the most keys
    const int nqt = (a.L + C::BMT - 1) / C::BMT;
    const int qt = nqt - 1 - blockIdx.x;
    const int kv = blockIdx.y / (G / C::HPW);
    const int hblk = blockIdx.y % (G / C::HPW);
    const int b = blockIdx.z;
    const int h = kv * G + hblk * C::HPW + wave % C::HPW;
    const int row0 = qt * C::BMT + (wave / C::HPW) * 32;    // first row of this wave
    const int wg_row_end = min(a.L, (qt + 1) * C::BMT);     // rows of the workgroup end here
    const int ntiles = (wg_row_end + C::BN - 1) / C::BN;    // causal key tiles of the workgroup

    // P V in float16 when a float16 copy of V exists and every V element fits
    // (the flag is uniform: the grid that does not match it exits here)
    constexpr bool f16pv = F16;
    if (a.vflag != nullptr && ((*a.vflag == 0u) != F16)) return;
    const uint16_t* kg = a.k + ((size_t)b * a.Hkv + kv) * (size_t)a.L * D;
    // V: row-major bfloat16, or the float16 V^T image (whole 64-key tiles)
    const int nimg = (a.L + C::BN - 1) / C::BN;
    const uint16_t* vg = f16pv ? a.v16 + ((size_t)b * a.Hkv + kv) * (size_t)nimg * (C::KTILE / 2)
                               : a.v + ((size_t)b * a.Hkv + kv) * (size_t)a.L * D;
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kg), 0, a.L * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(vg), 0, f16pv ? nimg * C::KTILE : a.L * D * 2, 0x00020000);

    // ---- Q^T fragments (B operand): query row row0 + 16 qb + l16, dims 32 s + 8 lq + e
    bf16x8 qf[2][C::KSTEPS];
    {
        const uint16_t* qg = a.q + ((size_t)b * a.Hq + h) * (size_t)a.L * D;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int r = min(row0 + 16 * qb + l16, a.L - 1);
#pragma unroll
            for (int s = 0; s < C::KSTEPS; ++s)
                qf[qb][s] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qg + (size_t)r * D + 32 * s + 8 * lq));
        }
    }

    // ---- K and V tile staging: each wave moves a quarter of the tile; source
    // offsets apply an XOR swizzle (16-byte chunk c of row r sits in slot
    // c ^ (r % CPR)) so that MFMA-layout reads are bank-conflict free
    constexpr int NVO = C::CPR / C::RPI > 0 ? C::CPR / C::RPI : 1;
    int vo[NVO];
#pragma unroll
    for (int j = 0; j < NVO; ++j) {
        const int row = j * C::RPI + lane / C::CPR;
        vo[j] = (lane / C::CPR) * (D * 2) + (((lane % C::CPR) ^ (row % C::CPR)) * 16);
    }
    auto issue_tile = [&](__amdgpu_buffer_rsrc_t rs, unsigned char* dst, int tile) {
#pragma unroll
        for (int i = 0; i < C::NLD; ++i) {
            const int li = wave * C::NLD + i;          // load instruction of the tile
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (__attribute__((address_space(3))) void*)(dst + li * 1024), 16,
                vo[li % NVO], (tile * C::BN + li * C::RPI) * (D * 2), 0, 0);
        }
    };
    auto issue_k = [&](int tile, int slot) { issue_tile(krs, s_kv[slot], tile); };
    // a V^T image tile is already laid out as in LDS: a straight copy
    auto issue_vimg = [&](int tile, int buf) {
#pragma unroll
        for (int i = 0; i < C::NLD; ++i) {
            const int li = wave * C::NLD + i;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                vrs, (__attribute__((address_space(3))) void*)(s_kv[2 + buf] + li * 1024), 16,
                lane * 16, tile * C::KTILE + li * 1024, 0, 0);
        }
    };
    auto issue_v = [&](int tile, int buf) {
        if constexpr (f16pv) issue_vimg(tile, buf);
        else issue_tile(vrs, s_kv[2 + buf], tile);
    };
    // S^T block (keys 16 kb + 4 lq + r, query rows 16 qb + l16) of one K tile
    auto scores = [&](int buf, f32x4 (&st)[2][4]) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int key = 16 * kb + l16;              // A operand row: key of the tile
            const unsigned char* srow = &s_kv[buf][((key / C::RPI) * 64 + (key % C::RPI) * C::CPR) * 16];
            const int swz = key % C::CPR;
            f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < C::KSTEPS; ++s) {
                const int c = 4 * s + lq;               // dims 32 s + 8 lq .. + 7
                const bf16x8 kf = __builtin_bit_cast(bf16x8, *(const u32x4*)(srow + (c ^ swz) * 16));
                acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[0][s], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[1][s], acc1, 0, 0, 0);
            }
            st[0][kb] = acc0;
            st[1][kb] = acc1;
        }
        // the K fragments of key block kb+1 are read while kb's MFMAs run
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * C::KSTEPS, 0);
#pragma unroll
        for (int kb = 0; kb < 3; ++kb) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * C::KSTEPS, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, C::KSTEPS, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * C::KSTEPS, 0);
    };

    // ======================= sweep A: row log-sum-exp =========================
    // K tiles go three ahead through the four slots: at step j the loads of
    // tiles j+1 and j+2 may still be in flight (loads retire in issue order,
    // so waiting until at most their count is outstanding completes tile j).
    // Each lane sums exp2(scale (s - m)) against a reference m that is a score
    // it has seen (so the sum is at least 1 and every term is positive: no
    // cancellation, whatever m is).  The tile maximum is only taken when the
    // tile's sum is not finite or above 2^64: on the first tile (m = -inf) and
    // when a score lies 64 or more above m in exp2 units.
    float m_l[2] = {NEG_INF, NEG_INF}, l_l[2] = {0.f, 0.f};
    float nmc_l[2] = {INFINITY, INFINITY};                 // -m * xscale
    if constexpr (!PRE) {
        issue_k(0, 0);
        if (ntiles > 1) issue_k(1, 1);
        if (ntiles > 2) issue_k(2, 2);
    }
    for (int j = 0; j < (PRE ? 0 : ntiles); ++j) {
        const int ahead = ntiles - 1 - j;
        if (ahead >= 2) pf_wait_vmem_n<2 * C::NLD>();
        else if (ahead == 1) pf_wait_vmem_n<C::NLD>();
        else pf_wait_vmem();
        __syncthreads();                                   // tile j complete; tile j-1 no longer read
        if (j + 3 < ntiles) issue_k(j + 3, (j + 3) & 3);
        f32x4 st[2][4];
        scores(j & 3, st);
        // statistics in raw score units (the scale is positive); only tiles
        // that cross the diagonal mask
        const bool diag = j * C::BN + C::BN - 1 > row0;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int row = row0 + 16 * qb + l16;
            if (diag) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (j * C::BN + 16 * kb + 4 * lq + r > row) st[qb][kb][r] = NEG_INF;
            }
            float sum = 0.f;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) sum += pf_exp2(fmaf(st[qb][kb][r], a.xscale, nmc_l[qb]));
            if (!(sum <= 0x1p64f)) {                       // also NaN: m = -inf meets a masked score
                float tmax = NEG_INF;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, st[qb][kb][r]);
                const float mn = fmaxf(m_l[qb], tmax);
                sum = 0.f;
                if (mn != NEG_INF) {                       // else no score of this lane yet
                    const float nmc = -mn * a.xscale;
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) sum += pf_exp2(fmaf(st[qb][kb][r], a.xscale, nmc));
                    l_l[qb] *= pf_exp2((m_l[qb] - mn) * a.xscale);     // 0 while m = -inf (l = 0)
                    m_l[qb] = mn;
                    nmc_l[qb] = nmc;
                }
            }
            l_l[qb] += sum;
        }
    }
    // the four lanes of a row (16 lanes apart) hold partial statistics
    float lse2[2], thr[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        if constexpr (PRE) {
            // keep a >= theta  <=>  raw >= theta / scale; -inf keeps every valid element
            const int row = min(row0 + 16 * qb + l16, a.L - 1);
            const float th = a.theta[(size_t)h * a.n_rows + min(row, a.n_rows - 1)];
            thr[qb] = fmaxf(th / a.scale, -3.402823466e38f);
            lse2[qb] = 0.f;
            continue;
        }
        float M = m_l[qb];                                 // raw units
        M = fmaxf(M, __shfl_xor(M, 16));
        M = fmaxf(M, __shfl_xor(M, 32));
        float part = (m_l[qb] == NEG_INF) ? 0.f : l_l[qb] * pf_exp2((m_l[qb] - M) * a.xscale);
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        lse2[qb] = M * a.xscale + __log2f(part);           // log2 domain
        const int row = min(row0 + 16 * qb + l16, a.L - 1);
        const float th = a.theta[(size_t)h * a.n_rows + min(row, a.n_rows - 1)];
        // keep  s >= theta  <=>  scale * raw >= log2(theta) + lse2; compared in raw
        // units; the clamp keeps masked (-inf) elements out when theta keeps all
        thr[qb] = fmaxf(log2_threshold(th, lse2[qb]) / a.xscale, -3.402823466e38f);
    }

    // ================ sweep B: threshold, exact SDC, P V on MFMA ===============
    f32x4 o[2][C::DB];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int db = 0; db < C::DB; ++db) o[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    int cnt[2] = {0, 0};
    float mass[2] = {0.f, 0.f};
    // PRE: reference maximum (raw units, lags the true one by < 8 / xscale),
    // true row maximum, and the sum over all elements, all row-uniform frames
    float mref[2] = {NEG_INF, NEG_INF}, mtop[2] = {NEG_INF, NEG_INF}, lall[2] = {0.f, 0.f};
    unsigned char* kmask = MASK ? a.kept_mask + ((size_t)b * a.Hq + h) * (size_t)a.L * a.L : nullptr;

    // V^T fragments (A operand of O^T += V^T P^T) come straight from the
    // row-major V tile with LDS transpose reads: in each 16-lane group, lane i
    // receives column i % 4 of the 8-byte rows addressed by lanes i / 4 + 4 e,
    // e = 0..3.  Lane r of group lq points at V[key(r / 4)][16 db + 4 (r % 4)],
    // so lane i gets V[key(e)][16 db + i] for four keys.  The keys of k-slot j
    // follow the P^T fragment: 32 ks + 16 (j / 4) + 4 lq + j % 4.
    int vtr_off[2];                                        // byte offsets for j / 4 = 0, 1, db = 0
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int key = 16 * hh + 4 * lq + l16 / 4;        // plus 32 ks: same residue mod CPR
        const int c = (4 * (l16 % 4)) / 8;                 // 16-byte chunk of dims 4 (l16 % 4) .. + 3
        vtr_off[hh] = key * (D * 2) + ((c ^ (key % C::CPR)) * 16) + ((l16 % 4) & 1) * 8;
    }
    auto vt_frag = [&](int buf, int ks, int db) -> bf16x8 {
        // chunk index of dims 16 db + ... is 2 db + c; the swizzle XORs the chunk
        // index with key % CPR, and 2 db only touches bits that c does not use
        const unsigned char* base = &s_kv[2 + buf][32 * ks * (D * 2)];
        const int dboff = (2 * db) * 16;
        const pf_i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) pf_i16x4*)(base + (vtr_off[0] ^ dboff)));
        const pf_i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) pf_i16x4*)(base + (vtr_off[1] ^ dboff)));
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        const i16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8, both);
    };

    // float16 form: V^T fragments are single 16-byte reads of the image tile.
    // Dimension row d (VROW bytes) holds the tile's keys in P^T fragment
    // order (position 32 h + 8 q + e holds key 32 h + 16 (e / 4) + 4 q + e % 4),
    // 16-byte chunk c in slot c ^ (d % 8) ^ ((d / 8) % 2), so that any 16
    // consecutive dimensions at one chunk fall in 16 distinct 16-byte bank
    // groups.  Lane (l16, lq) reads dimension 16 db + l16, chunk 4 ks + lq.
    int vimg_off[2];
    {
        const int sw = (l16 & 7) ^ ((l16 >> 3) & 1);
        vimg_off[0] = l16 * C::VROW + ((lq ^ sw) * 16);
        vimg_off[1] = vimg_off[0] ^ 64;                     // chunk 4 + lq: bit 2 of the chunk flips
    }
    auto vt_frag16 = [&](int buf, int ks, int db) -> pf_f16x8 {
        return __builtin_bit_cast(pf_f16x8,
                                  *(const u32x4*)&s_kv[2 + buf][vimg_off[ks] + db * 16 * C::VROW]);
    };

    if constexpr (!PRE) __syncthreads();                   // sweep A is done with both K buffers
    issue_k(0, 0);
    issue_v(0, 0);
    // tile j lives in buffer j & 1; the loop takes two tiles per trip so that
    // the buffer is a constant in each half and its LDS base folds into the
    // read instructions' offsets
    auto step_b = [&](int j, auto buf_c) {
        constexpr int buf = decltype(buf_c)::value;
        pf_wait_vmem();
        __syncthreads();                                   // K, V tile j landed; tile j-1 fully used
        if (j + 1 < ntiles) { issue_k(j + 1, 1 - buf); issue_v(j + 1, 1 - buf); }
        f32x4 st[2][4];
        scores(buf, st);
        const bool diag = j * C::BN + C::BN - 1 > row0;
        unsigned pk[2][4][2], pl[2][4][2];                 // P^T fragments, packed bf16 (hi, lo)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int row = row0 + 16 * qb + l16;
            if (diag) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (j * C::BN + 16 * kb + 4 * lq + r > row) st[qb][kb][r] = NEG_INF;
            }
            if (MASK && row < a.L) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int key = j * C::BN + 16 * kb + 4 * lq + r;
                        if (key <= row) kmask[(size_t)row * a.L + key] = st[qb][kb][r] >= thr[qb] ? 1 : 0;
                    }
            }
            // float16 P V: weights scaled by 2^PSC (see the file header)
            float nlse = -lse2[qb] + (float)PSC;
            if constexpr (PRE) {
                float tmax = NEG_INF;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, st[qb][kb][r]);
                tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
                tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
                mtop[qb] = fmaxf(mtop[qb], tmax);
                if ((tmax - mref[qb]) * a.xscale > 8.f) {         // also the first tile (mref = -inf)
                    const float f = pf_exp2((mref[qb] - tmax) * a.xscale);
#pragma unroll
                    for (int db = 0; db < C::DB; ++db)
#pragma unroll
                        for (int r = 0; r < 4; ++r) o[qb][db][r] *= f;
                    lall[qb] *= f;
                    mass[qb] *= f;
                    mref[qb] = tmax;
                }
                nlse = (mref[qb] == NEG_INF ? 0.f : -mref[qb] * a.xscale) + (float)PSC;
            }
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                float p[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool kp = st[qb][kb][r] >= thr[qb];
                    if constexpr (PRE) {
                        const float e = pf_exp2(fmaf(st[qb][kb][r], a.xscale, nlse));
                        lall[qb] += e;
                        p[r] = kp ? e : 0.f;
                    } else {
                        p[r] = kp ? pf_exp2(fmaf(st[qb][kb][r], a.xscale, nlse)) : 0.f;
                    }
                    cnt[qb] += kp ? 1 : 0;
                    if constexpr (MASS) mass[qb] += p[r];
                }
                if constexpr (f16pv) {
                    pk[qb][kb][0] = pack_f16x2(p[0], p[1]);
                    pk[qb][kb][1] = pack_f16x2(p[2], p[3]);
                } else {
                    split_bf16x2(p[0], p[1], pk[qb][kb][0], pl[qb][kb][0]);
                    split_bf16x2(p[2], p[3], pk[qb][kb][1], pl[qb][kb][1]);
                }
            }
        }
        // O^T += V^T P^T over 32 keys per step; each V^T fragment serves both row blocks
        if constexpr (f16pv) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                pf_f16x8 pb[2];
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    const u32x4 pv = {pk[qb][2 * ks][0], pk[qb][2 * ks][1], pk[qb][2 * ks + 1][0], pk[qb][2 * ks + 1][1]};
                    pb[qb] = __builtin_bit_cast(pf_f16x8, pv);
                }
#pragma unroll
                for (int db = 0; db < C::DB; ++db) {
                    const pf_f16x8 vtf = vt_frag16(buf, ks, db);
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb)
                        o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vtf, pb[qb], o[qb][db], 0, 0, 0);
                }
            }
            pf_ds_mfma_pipeline<1, 2, 0>();
            pf_ds_mfma_pipeline<2 * C::DB - 1, 1, 2>();
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            return;
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 pb[2], pbl[2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const u32x4 pv = {pk[qb][2 * ks][0], pk[qb][2 * ks][1], pk[qb][2 * ks + 1][0], pk[qb][2 * ks + 1][1]};
                const u32x4 pw = {pl[qb][2 * ks][0], pl[qb][2 * ks][1], pl[qb][2 * ks + 1][0], pl[qb][2 * ks + 1][1]};
                pb[qb] = __builtin_bit_cast(bf16x8, pv);
                pbl[qb] = __builtin_bit_cast(bf16x8, pw);
            }
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
                const bf16x8 vtf = vt_frag(buf, ks, db);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vtf, pb[qb], o[qb][db], 0, 0, 0);
                    o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vtf, pbl[qb], o[qb][db], 0, 0, 0);
                }
            }
        }
        // the V^T fragment of the next (ks, db) is read while the current one's MFMAs run
        pf_ds_mfma_pipeline<1, 4, 0>();
        pf_ds_mfma_pipeline<2 * C::DB - 1, 2, 4>();
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    };
    for (int j = 0; j < ntiles; j += 2) {
        step_b(j, std::integral_constant<int, 0>{});
        if (j + 1 < ntiles) step_b(j + 1, std::integral_constant<int, 1>{});
    }

    // ---- epilogue: row totals, SDC_NONE / VMC, output (weights, sums and
    // accumulators lose the 2^PSC of the float16 form first)
    const float unscale = 1.0f / (float)(1 << PSC);
    const bool renorm = (a.flags & 2u) != 0;
    const bool vmc = (a.flags & 1u) != 0 && !renorm;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        int c = cnt[qb];
        c += __shfl_xor(c, 16);
        c += __shfl_xor(c, 32);
        float m = mass[qb];
        m += __shfl_xor(m, 16);
        m += __shfl_xor(m, 32);
        m *= unscale;
        const int row = row0 + 16 * qb + l16;
        if (row >= a.L) continue;
        float bta = renorm ? 0.f : 1.f - m;
        float inv = (renorm && c > 0) ? 1.f / m : 1.f;
        if constexpr (PRE) {
            // Eq. 4: kept weights exp(a - max) / (R + E~), all in the frame mref
            float l = lall[qb];
            l += __shfl_xor(l, 16);
            l += __shfl_xor(l, 32);
            l *= unscale;
            const int rid = min(row, a.n_rows - 1);
            float den;
            if (renorm) den = m;
            else if (a.flags & kFlagExpth)           // gamma (n - k~) e^(theta - a_ref)
                den = m + a.gamma * (float)(row + 1 - c) *
                              pf_exp2(a.theta[(size_t)h * a.n_rows + rid] * kLog2e - mref[qb] * a.xscale);
            else if (a.flags & kFlagOffline)         // E~ is relative to the true row maximum
                den = m + a.e_tilde[(size_t)h * a.n_rows + rid] * pf_exp2((mtop[qb] - mref[qb]) * a.xscale);
            else den = l;                            // exact: R + E
            const bool ok = den > 0.f && !(renorm && c == 0);
            inv = ok ? 1.f / den : 0.f;
            bta = (ok && !renorm) ? 1.f - m * inv : 0.f;
        }
        const float* mu = vmc ? a.mu + (((size_t)b * a.Hkv + kv) * (size_t)a.L + row) * D : nullptr;
        if (lq == 0) {
            const size_t ro = ((size_t)b * a.Hq + h) * (size_t)a.L + row;
            if (a.kept_count) a.kept_count[ro] = c;
            if (a.beta) a.beta[ro] = bta;
        }
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
            float y[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int dim = 16 * db + 4 * lq + r;
                float v = o[qb][db][r] * unscale;
                if (PRE || renorm) v = c > 0 ? v * inv : 0.f;
                if (vmc) v = fmaf(bta, mu[dim], v);
                y[r] = v;
            }
            const size_t oi = ((((size_t)b * a.Hq + h) * (size_t)a.L) + row) * D + 16 * db + 4 * lq;
            if (a.flags & kFlagOutF32) {
                *(float4*)((float*)a.out + oi) = make_float4(y[0], y[1], y[2], y[3]);
            } else {
                *(uint2*)(a.out + oi) = make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
            }
        }
    }
#endif
}

// The float16 V^T image of one 64-key tile of one (sequence, KV head), in the
// layout the prefill kernel's LDS tile has (see vt_frag16 there): keys past L
// are zero.  The tile goes through LDS (rows padded by one word, so that the
// eight keys of one output chunk sit in distinct banks); any element beyond
// 16 in magnitude, or not finite, sets *flag (every writer stores the same
// value).  One workgroup per (sequence and KV head, tile), tile fastest;
// 256 threads.
template <int D>
__global__ __launch_bounds__(256) void v_to_f16t_kernel(const uint16_t* v, int L, uint16_t* img, unsigned* flag) {
    constexpr int PW = D / 2 + 1;                        // words per LDS row (bf16 pairs + pad)
    constexpr int CPR = D / 8;                           // 16-byte chunks per V row
    constexpr int NCH = 64 * D / 8;                      // 16-byte chunks per tile
    __shared__ unsigned s_v[64 * PW];
    const int nimg = (L + 63) / 64;
    const int t = (int)(blockIdx.x % (unsigned)nimg);
    const size_t bkv = blockIdx.x / (unsigned)nimg;
    const uint16_t* vt = v + (bkv * (size_t)L + (size_t)t * 64) * D;
    for (int idx = threadIdx.x; idx < NCH; idx += 256) {
        const int key = idx / CPR, part = idx % CPR;
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (t * 64 + key < L) raw = *(const u32x4*)(vt + (size_t)key * D + 8 * part);
#pragma unroll
        for (int w = 0; w < 4; ++w) s_v[key * PW + 4 * part + w] = raw[w];
    }
    __syncthreads();
    uint16_t* it = img + (bkv * (size_t)nimg + t) * (size_t)(64 * D);
    bool bad = false;
    for (int q = threadIdx.x; q < NCH; q += 256) {
        const int d = q / 8, slot = q % 8;
        const int c = slot ^ (d & 7) ^ ((d >> 3) & 1);   // chunk held in this slot
        const int h = c / 4, qq = c % 4;                 // positions 32 h + 8 qq + e
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int key = 32 * h + 16 * (e / 4) + 4 * qq + e % 4;
            const unsigned wd = s_v[key * PW + d / 2];
            x[e] = __uint_as_float((d & 1) ? (wd & 0xffff0000u) : (wd << 16));
            bad |= !(fabsf(x[e]) <= 16.0f);
        }
        u32x4 o;
#pragma unroll
        for (int w = 0; w < 4; ++w) o[w] = pack_f16x2(x[2 * w], x[2 * w + 1]);
        *(u32x4*)(it + 8 * q) = o;
    }
    if (bad) *flag = 1u;
}

// ------------------------------------------------------------------ host side
int launch_prefix_mean(const void* v, int groups, int L, int d, int dtype, float* mu, hipStream_t s);

bool prefill_bf16_supported(int d, int G) {
    return (d == 64 || d == 128) && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
}

template <int D, int G, bool PRE, bool F16, bool MASS>
static void launch_form(const PrefillKArgs& a, dim3 grid, hipStream_t s) {
    if (a.kept_mask) hipLaunchKernelGGL((prefill_bf16_kernel<D, G, true, PRE, F16, MASS>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((prefill_bf16_kernel<D, G, false, PRE, F16, MASS>), grid, dim3(256), 0, s, a);
}

template <int D, int G, bool F16>
static void launch_pv_form(const PrefillKArgs& a, dim3 grid, hipStream_t s, bool pre, bool mass) {
    if (pre) launch_form<D, G, true, F16, true>(a, grid, s);
    else if (mass) launch_form<D, G, false, F16, true>(a, grid, s);
    else launch_form<D, G, false, F16, false>(a, grid, s);
}

template <int D, int G>
static int launch_prefill_variant(const PrefillKArgs& a, hipStream_t s) {
    using C = PrefillCfg<D, G>;
    const dim3 grid((a.L + C::BMT - 1) / C::BMT, a.Hkv * (G / C::HPW), a.B);
    // the variant that also writes the kept mask is only used when one is asked
    // for; with a float16 copy of V both P V forms are launched (one exits)
    const bool pre = (a.flags & kFlagPre) != 0;
    const bool mass = pre || (a.flags & (kFlagVmc | kFlagNone)) != 0 || a.beta != nullptr;
    if (a.v16) {
        launch_pv_form<D, G, true>(a, grid, s, pre, mass);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    launch_pv_form<D, G, false>(a, grid, s, pre, mass);
    return hipGetLastError();
}

template <int D>
static int launch_prefill_d(const PrefillKArgs& a, int G, hipStream_t s) {
    switch (G) {
        case 1: return launch_prefill_variant<D, 1>(a, s);
        case 2: return launch_prefill_variant<D, 2>(a, s);
        case 4: return launch_prefill_variant<D, 4>(a, s);
        case 8: return launch_prefill_variant<D, 8>(a, s);
        default: return launch_prefill_variant<D, 16>(a, s);
    }
}

size_t prefill_mu_bytes(int B, int Hkv, int L, int d) { return (size_t)B * Hkv * L * d * sizeof(float); }
// the float16 V^T image: whole 64-key tiles
size_t prefill_v16_bytes(int B, int Hkv, int L, int d) {
    return (size_t)B * Hkv * (size_t)((L + 63) / 64) * 64 * d * sizeof(uint16_t);
}

int launch_prefill_bf16(const PrefillParams& p, float* mu_ws, hipStream_t s) {
    const bool vmc = (p.flags & 1u) && !(p.flags & 2u);
    if (vmc) {
        const int e = launch_prefix_mean(p.v, p.B * p.Hkv, p.L, p.d, p.dtype, mu_ws, s);
        if (e != hipSuccess) return e;
    }
    // workspace: [prefix means][float16 V][flag]; the float16 P V path needs all of it
    const size_t mu_b = (prefill_mu_bytes(p.B, p.Hkv, p.L, p.d) + 255) & ~(size_t)255;
    const size_t v16_b = (prefill_v16_bytes(p.B, p.Hkv, p.L, p.d) + 255) & ~(size_t)255;
    uint16_t* v16 = nullptr;
    unsigned* vflag = nullptr;
    if (p.ws && p.ws_bytes >= mu_b + v16_b + 256) {
        v16 = (uint16_t*)((char*)p.ws + mu_b);
        vflag = (unsigned*)((char*)p.ws + mu_b + v16_b);
        int e = launch_fill_u32(vflag, 4, 0u, s);
        if (e != hipSuccess) return e;
        const dim3 grid((unsigned)((size_t)((p.L + 63) / 64) * p.B * p.Hkv));
        if (p.d == 64) hipLaunchKernelGGL(v_to_f16t_kernel<64>, grid, dim3(256), 0, s, (const uint16_t*)p.v, p.L, v16, vflag);
        else hipLaunchKernelGGL(v_to_f16t_kernel<128>, grid, dim3(256), 0, s, (const uint16_t*)p.v, p.L, v16, vflag);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    PrefillKArgs a = {};
    a.q = (const uint16_t*)p.q; a.k = (const uint16_t*)p.k; a.v = (const uint16_t*)p.v;
    a.theta = p.theta; a.mu = vmc ? mu_ws : nullptr;
    a.out = (uint16_t*)p.out; a.kept_count = p.kept_count; a.beta = p.beta; a.kept_mask = p.kept_mask;
    a.B = p.B; a.Hq = p.Hq; a.Hkv = p.Hkv; a.L = p.L; a.n_rows = p.n_rows;
    a.xscale = p.scale * kLog2e;
    a.flags = p.flags;
    a.scale = p.scale;
    a.e_tilde = p.e_tilde;
    a.gamma = p.gamma;
    a.v16 = v16;
    a.vflag = vflag;
    const int G = p.Hq / p.Hkv;
    return p.d == 64 ? launch_prefill_d<64>(a, G, s) : launch_prefill_d<128>(a, G, s);
}

}  // namespace topth
