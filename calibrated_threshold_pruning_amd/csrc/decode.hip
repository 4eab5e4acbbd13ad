// Top-theta decode for bfloat16 KV caches on gfx950.
//
// One generative-decoding step ("Top-Theta Attention: Sparsifying Transformers
// by Compensated Thresholding", Sec. 2.2 decode phase): every query head scores
// all n cached keys, keeps the post-softmax elements s_j >= theta (Sec. 3),
// weights them by s_j itself (exact SDC, Sec. 3.2.1 Eq. 4), adds beta * mu
// (VMC, Sec. 3.2.2 Eq. 5-7), and -- the point of the method in decoding -- only
// the V rows that some head of the GQA group keeps are read (Sec. 4.6).
//
// Kernel shape (persistent; the grid never exceeds the resident capacity):
//   work item = (group = (b, kv head), chunk of keys); one workgroup of 8 waves
//   per CU.
//   Phase 1  each wave stages its keys' K rows in LDS (buffer_load ... lds,
//            XOR-swizzled) and forms the g scores per key with
//            v_mfma_f32_16x16x32_bf16 (query heads in the A operand, several
//            key tiles packed into the 16 rows when g < 16).  Scores stay in
//            registers; the wave and the workgroup reduce per-head (max, sum
//            of exp2) and publish them.
//   Exchange every chunk of a group publishes its per-head (max, sum of exp2)
//            to a workspace slot and polls all of the group's slots; each then
//            merges them in chunk order, so all see the same row log-sum-exp.
//   Phase 2  compare x >= log2(theta) + lse2 per (key, head); OR over the
//            group's heads; ballot prefix sums compact the kept keys into a
//            per-wave LDS list; only those V rows are gathered (buffer_load ...
//            lds) and O^T += V^T W runs on MFMA from LDS transpose reads.
//   Combine  chunk 0 of each group polls the other chunks' partial outputs,
//            sums them in chunk order, applies beta * mu and empties the slots.
// Reductions never use float atomics, so results are run-to-run identical.
#include "topth_internal.h"

#include <math.h>

#include <algorithm>

namespace topth {

struct DecodeKArgs {
    const uint16_t* q; const uint16_t* k; const uint16_t* v; const int* seq_lens;
    const float* theta; const float* v_mean;
    uint16_t* out; int* kept_count; float* beta; int* vrows_read; unsigned char* kept_mask;
    int* status;       // workspace header: word 0 the status, word 1 the spin limit (0: default)
    // exchange slots, kWsSlotEmpty until published: (max, sum of exp2) per chunk
    // and head as one 64-bit word, and the partial outputs of chunks 1.. for chunk 0
    unsigned long long* part_ml; float* part_out; float* part_mass; int* part_cnt; int* part_union;
    float* ovf_w;      // weights of kept keys that do not fit the LDS list, [B*Hkv*Lmax][GW]
    int B, Hq, Hkv, Lmax, n_rows, chunks, items;
    float xscale;
    unsigned flags;
    int xcd_map;       // 1: chunks of a group on one XCD (grid and items multiples of 8 * chunks)
    const float* e_tilde;   // pre-softmax offline estimate of E~ [Hq][n_rows], or NULL
    float gamma;            // pre-softmax exp-threshold estimate
    int min_votes;          // GQA: load a key when at least this many heads keep it (<= 1: any)
    int augment;            // GQA: every head uses all loaded keys, not only its own
    // running V mean to update in place (the mean of rows 0..n-2 becomes that of
    // rows 0..n-1) and to use for VMC; NULL: v_mean is used as given
    float* v_mean_append;
};

// One workgroup of kDecodeWaves waves per CU: two workgroups on a CU stream at
// different rates (the older one's loads are served first), which leaves the
// chunks on the second one, and their groups, behind.
constexpr int kDecodeWaves = 8;

template <int D, int G, int NT>
struct DecodeCfg {
    static constexpr int P = (G <= 4) ? 4 : (G == 8 ? 2 : 1);  // key tiles packed per MFMA
    static constexpr int GP = 16 / P;          // A-operand rows per key tile (heads, padded)
    static constexpr int BPT = 4 / P;          // 16-lane blocks per key tile
    static constexpr int KT = 16 * P;          // keys per wave tile
    static constexpr int STEPS = D * P / 32;   // MFMA steps over the head dimension
    static constexpr int WAVES = kDecodeWaves;
    static constexpr int THREADS = WAVES * 64;
    static constexpr int KEYS_PER_WG = WAVES * NT * KT;
    static constexpr int GW = G < 4 ? 4 : G;   // heads per LDS weight row (padded to 4)
    static constexpr int LPR = G <= 4 ? 16 : 32;  // lanes per V row in the gather
    static constexpr int RPG = 64 / LPR;       // V rows per wave gather instruction
    static constexpr int DPL = D / LPR;        // V dims per lane in the gather
    static constexpr int WKEYS = NT * KT;      // keys of one wave
    static constexpr int CPR = D / 8;          // 16-byte chunks per K row
    static constexpr int RPI = 64 / CPR;       // K rows per wave load instruction
    static constexpr int NLD = KT / RPI;       // load instructions per wave tile
    static constexpr int STAGE_BYTES = KT * D * 2;              // one staged wave tile
    static constexpr int NBUF = P == 4 ? 1 : 2;                 // stage buffers per wave
    // the weighted V sum runs on MFMA in batches of 32 rows where the stage
    // holds such a batch next to a useful weight list (every group size but 16)
    static constexpr bool MFMA_ACC = NBUF * STAGE_BYTES >= 32 * D * 2 + 4096;
    static constexpr int DB = D / 16;                           // 16-dim blocks of the output
    static constexpr int CAPW = (NBUF * STAGE_BYTES - (MFMA_ACC ? 32 * D * 2 : 4096)) / (GW * 4);  // kept-key weights in LDS per wave
    static constexpr int RED_BYTES = WAVES * G * D * 4;         // output partials per workgroup
    static constexpr int KBUF_BYTES =
        WAVES * NBUF * STAGE_BYTES > RED_BYTES ? WAVES * NBUF * STAGE_BYTES : RED_BYTES;
    static_assert(STEPS >= 1 && NLD >= 1, "head dimension too small");
    static_assert(WKEYS <= 65536, "wave key offsets must fit 16 bits");
    static_assert(NT <= 32, "one bit per tile in a 32-bit mask");
    // spare list slots (one per lane) for stores that keep nothing
    static constexpr int SPARE = CAPW < WKEYS ? CAPW : WKEYS;
    static_assert((SPARE + 64) * GW * 4 <= NBUF * STAGE_BYTES, "spare weight rows inside the stage");
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Cross-workgroup data of one group (partials written by one chunk, read by the
// others) moves through agent-scope atomic stores and loads: they are coherent
// across the XCDs' separate L2 caches without the L2 write-back and invalidate
// that a device-wide fence costs.  Every published word is one store, and a
// reader polls the word itself until it no longer holds the empty pattern, so
// no counter or fence orders them.
__device__ __forceinline__ void publish(float* p, float v) {
    __hip_atomic_store(reinterpret_cast<unsigned*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish_i(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float consume(const float* p) {
    return __uint_as_float(__hip_atomic_load(reinterpret_cast<const unsigned*>(p), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT));
}
// Exchange slots hold kWsSlotEmpty (in every 32-bit word) until their chunk
// publishes them.  A reader issues the loads of up to eight slots together and
// re-polls the ones still empty; the combining chunk, the last reader of every
// slot of its group, sets each slot back to empty.
constexpr unsigned long long kSlot64Empty = ((unsigned long long)kWsSlotEmpty << 32) | kWsSlotEmpty;
__device__ __forceinline__ unsigned long long load64(const unsigned long long* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned load32(const void* p) {
    return __hip_atomic_load(reinterpret_cast<const unsigned*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store32(void* p, unsigned v) {
    __hip_atomic_store(reinterpret_cast<unsigned*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A bounded wait: after `limit` polls that still find the slot empty it gives
// up, sets the status bit in the workspace header and raises `failed`; the
// caller's group then reports poisoned outputs instead of partial sums.
__device__ __forceinline__ unsigned long long wait_slot64(const unsigned long long* p, unsigned long long v,
                                                        unsigned limit, int* status, bool& failed) {
    for (unsigned spins = 0; v == kSlot64Empty; v = load64(p)) {
        if (spins++ >= limit) { atomicOr(status, kStatusSpinTimeout); failed = true; break; }
        __builtin_amdgcn_s_sleep(1);
    }
    return v;
}
__device__ __forceinline__ unsigned wait_slot32(const void* p, unsigned v, unsigned limit, int* status,
                                                bool& failed) {
    for (unsigned spins = 0; v == kWsSlotEmpty; v = load32(p)) {
        if (spins++ >= limit) { atomicOr(status, kStatusSpinTimeout); failed = true; break; }
        __builtin_amdgcn_s_sleep(1);
    }
    return v;
}
// first + base[c * stride] for c = 1 .. n-1, added in order of c (float or int
// words); every slot read is set back to empty
template <typename T>
__device__ __forceinline__ T gather_chunks(T* base, size_t stride, int n, T first, unsigned limit,
                                           int* status, bool& failed) {
    T x = first;
    for (int c0 = 1; c0 < n; c0 += 8) {
        unsigned v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = (c0 + u < n) ? load32(base + (size_t)(c0 + u) * stride) : 0u;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (c0 + u < n) {
                T* p = base + (size_t)(c0 + u) * stride;
                x += __builtin_bit_cast(T, wait_slot32(p, v[u], limit, status, failed));
                store32(p, kWsSlotEmpty);
            }
        }
    }
    return x;
}
// The union sizes of chunks 1.. in chunk order; a chunk whose own waits gave
// up publishes -1 - (its union size), which marks the group as failed.
__device__ __forceinline__ int gather_union(int* base, int n, int first, unsigned limit, int* status,
                                            bool& failed) {
    int x = first;
    for (int c0 = 1; c0 < n; c0 += 8) {
        unsigned v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = (c0 + u < n) ? load32(base + c0 + u) : 0u;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (c0 + u < n) {
                int w = (int)wait_slot32(base + c0 + u, v[u], limit, status, failed);
                if (w < 0) { failed = true; w = -1 - w; }
                x += w;
                store32(base + c0 + u, kWsSlotEmpty);
            }
        }
    }
    return x;
}

// Default number of polls of one exchange slot before a wait gives up (each
// poll sleeps about 64 clocks: some 0.1 s in all); the workspace header can
// lower it.
constexpr unsigned kDefaultSpinLimit = 1u << 22;

// Outputs of a group whose exchange did not complete: NaN outputs and beta,
// -1 kept counts and V-row count.  The kept mask is left as it is.
template <int D, int G>
__device__ __forceinline__ void poison_group(const DecodeKArgs& a, int b, int kv, int group, int tid,
                                             int nthreads) {
    const size_t o0 = ((size_t)b * a.Hq + (size_t)kv * G) * D;
    for (int idx = tid; idx < G * D; idx += nthreads) {
        if (a.flags & kFlagOutF32) ((float*)a.out)[o0 + idx] = __uint_as_float(0x7FC00000u);
        else a.out[o0 + idx] = 0x7FC0u;                                    // bfloat16 NaN
    }
    if (tid < G) {
        const size_t o = (size_t)b * a.Hq + (size_t)kv * G + tid;
        if (a.kept_count) a.kept_count[o] = -1;
        if (a.beta) a.beta[o] = __uint_as_float(0x7FC00000u);
    }
    if (tid == 0 && a.vrows_read) a.vrows_read[group] = -1;
}

// Bit-sliced vote counts: plane i holds bit i of one count per tile bit.
// votes_add adds a 0/1 mask; votes_merge adds the counts of the lane `o` lanes
// away; votes_at_least gives the tiles whose count is >= m (m uniform).
__device__ __forceinline__ void votes_add(unsigned (&pl)[5], unsigned m) {
    unsigned carry = m;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const unsigned c = pl[i] & carry;
        pl[i] ^= carry;
        carry = c;
    }
}
__device__ __forceinline__ void votes_merge(unsigned (&pl)[5], int o) {
    unsigned q[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) q[i] = __shfl_xor(pl[i], o);
    unsigned carry = 0u;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const unsigned s = pl[i] ^ q[i] ^ carry;
        carry = (pl[i] & q[i]) | (carry & (pl[i] ^ q[i]));
        pl[i] = s;
    }
}
__device__ __forceinline__ unsigned votes_at_least(const unsigned (&pl)[5], int m) {
    if (m > 31) return 0u;                        // more than any group's heads
    unsigned gt = 0u, eq = ~0u;
#pragma unroll
    for (int i = 4; i >= 0; --i) {
        if ((m >> i) & 1) {
            eq &= pl[i];
        } else {
            gt |= eq & pl[i];
            eq &= ~pl[i];
        }
    }
    return gt | eq;
}

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0,15:14], expcnt[6:4], lgkmcnt[11:8])
// v_exp_f32 as is: results below the normal range flush to zero, which only
// affects probabilities under 2^-126.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }   // lgkmcnt(0)
template <int N>
__device__ __forceinline__ void wait_vmem_n() {                                          // vmcnt(N)
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x0F70);
}

template <int DPL> struct VVec;
template <> struct VVec<8> {
    typedef u32x4 T;
    static __device__ __forceinline__ T load(__amdgpu_buffer_rsrc_t r, int vo, int so) {
        return __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, 0);
    }
};
template <> struct VVec<4> {
    typedef uint2 T;
    static __device__ __forceinline__ T load(__amdgpu_buffer_rsrc_t r, int vo, int so) {
        typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u2;
        const u2 v = __builtin_amdgcn_raw_buffer_load_b64(r, vo, so, 0);
        return make_uint2(v[0], v[1]);
    }
};
template <> struct VVec<2> {
    typedef unsigned T;
    static __device__ __forceinline__ T load(__amdgpu_buffer_rsrc_t r, int vo, int so) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, vo, so, 0);
    }
};

typedef short dec_i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 dec_bf16x2 __attribute__((ext_vector_type(2)));
typedef float dec_f32x2 __attribute__((ext_vector_type(2)));
// (a, b) = hi + lo with both parts packed bfloat16 pairs (round to nearest even):
// the weights keep about 16 significant bits through the two bf16 MFMAs
__device__ __forceinline__ void split_bf16x2_pair(float a, float b, unsigned& hi, unsigned& lo) {
    const dec_f32x2 v = {a, b};
    hi = __builtin_bit_cast(unsigned, __builtin_convertvector(v, dec_bf16x2));
    const dec_f32x2 r = {a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u)};
    lo = __builtin_bit_cast(unsigned, __builtin_convertvector(r, dec_bf16x2));
}

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
__device__ __forceinline__ void unpack_bf16(const unsigned& u, float* f) {
    f[0] = __uint_as_float(u << 16); f[1] = __uint_as_float(u & 0xffff0000u);
}

// VOTE: the GQA selection variants (a key is loaded when at least min_votes
// heads keep it; augment gives every head all loaded keys); the plain
// per-head selection is compiled without them.
template <int D, int G, int NT, bool VOTE>
__global__ __launch_bounds__(kDecodeWaves * 64, 1) void decode_bf16_kernel(DecodeKArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)   // the host pass only needs the launch stub
    using C = DecodeCfg<D, G, NT>;
    // K tiles are staged through LDS: each wave loads its tile with 1 KiB
    // contiguous loads (16-byte chunks of a row permuted by an XOR swizzle) and
    // reads it back in the MFMA operand layout without bank conflicts.  After
    // phase 2 the same buffer holds the per-wave output partials.
    __shared__ __attribute__((aligned(16))) unsigned char s_kbuf[C::KBUF_BYTES];
    __shared__ __attribute__((aligned(16))) uint16_t s_q[G + 1][D + 8];   // row G stays zero
    __shared__ float s_m[C::WAVES][G], s_l[C::WAVES][G];
    __shared__ float s_T[G], s_lse[G], s_M[G];
    __shared__ unsigned short s_kl[C::WAVES][C::WKEYS + 64];   // kept keys of each wave (offsets from its base), + spare slots
    __shared__ float s_cm[C::WAVES][G];
    __shared__ int s_cc[C::WAVES][G];
    __shared__ int s_un[C::WAVES];
    __shared__ float s_mu[D];                  // the appended running mean of V
    __shared__ int s_fail;                     // some wait of this item gave up
    __shared__ int s_sticky;                   // the workspace status was already set at launch
    __shared__ unsigned s_limit;               // polls per exchange slot before a wait gives up

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int blk = lane >> 4;                 // 16-lane block of the MFMA operands
    const int cc = blk % C::BPT;               // block inside its key tile
    const int tt = blk / C::BPT;               // key tile of this lane
    const int mykey = (lane & 15) + 16 * tt;   // key of this lane inside a wave tile
    const int hb = 4 * cc;                     // first head of this lane's C registers
    const float NEG_INF = -INFINITY;
    unsigned char* stage = s_kbuf + wave * C::NBUF * C::STAGE_BYTES;
    float (*s_red)[G][D] = reinterpret_cast<float (*)[G][D]>(s_kbuf);

    // A-operand row of this lane: query head hi of key tile i / GP, or the zero row
    int qrow_lds;
    {
        const int i = lane & 15;
        const int hi = i % C::GP;
        qrow_lds = ((i / C::GP == tt) && (hi < G)) ? hi : G;
    }
    for (int t = tid; t < D + 8; t += C::THREADS) s_q[G][t] = 0;
    if (tid == 0) {
        // A workspace whose status is set may hold exchange slots that a late
        // chunk filled after its reader gave up: until topth_workspace_init
        // prepares it again, every call reports poisoned outputs.
        s_sticky = load32(a.status) != 0u;
        const unsigned lim = load32(a.status + 1);
        s_limit = lim != 0u ? lim : kDefaultSpinLimit;
    }
    __syncthreads();
    const unsigned spin_limit = s_limit;
    const bool sticky = s_sticky != 0;

    for (int slot = blockIdx.x; slot < a.items; slot += gridDim.x) {
        // Workgroups are dealt to the 8 XCDs round-robin by index; when the grid
        // allows it, all chunks of a group go to workgroups of one XCD so that
        // they stream under the same conditions and reach the exchange together.
        int item = slot;
        if (a.xcd_map) {
            const int per_xcd = gridDim.x / 8;
            const int round = slot / gridDim.x, r = slot % gridDim.x;
            item = round * gridDim.x + (r % 8) * per_xcd + r / 8;
        }
        const int group = item / a.chunks, chunk = item % a.chunks;
        const int b = group / a.Hkv, kv = group % a.Hkv;
        const int n = min(max(a.seq_lens[b], 1), a.Lmax);   // lengths outside [1, Lmax] are clamped
        const int wbase = chunk * C::KEYS_PER_WG + wave * NT * C::KT;
        if (sticky) {                          // uniform over the workgroup
            if (chunk == 0) {
                poison_group<D, G>(a, b, kv, group, tid, C::THREADS);
                if (a.v_mean_append != nullptr)
                    for (int dd = tid; dd < D; dd += C::THREADS) {
                        float* mu = a.v_mean_append + (size_t)group * D + dd;
                        const double prev = n > 1 ? (double)(n - 1) * (double)*mu : 0.0;
                        const double vn = (double)bf16_bits_to_f32(a.v[((size_t)group * a.Lmax + (n - 1)) * D + dd]);
                        *mu = (float)((prev + vn) / (double)n);
                    }
            }
            continue;
        }

        // ---- the group's query rows to LDS
        {
            const uint16_t* qg = a.q + ((size_t)b * a.Hq + (size_t)kv * G) * D;
            for (int idx = tid; idx < G * (D / 8); idx += C::THREADS) {
                const int h = idx / (D / 8), c = idx % (D / 8);
                *(u32x4*)&s_q[h][c * 8] = *(const u32x4*)(qg + (size_t)h * D + c * 8);
            }
        }
        __syncthreads();
        // every read of the previous item's flag came before the barrier above;
        // the first write of this item's comes after the next one
        if (tid == 0) s_fail = 0;

        // ---- phase 1: scores of this wave's keys, kept in registers
        // K of the group goes from HBM straight into this wave's LDS stage
        // (buffer_load ... lds, 1 KiB per instruction, four or eight whole rows);
        // the per-lane source offset applies the XOR swizzle, so the LDS slots
        // come out permuted for conflict-free MFMA-layout reads.  Rows past the
        // n valid keys read as zero (their scores are masked below).
        const uint16_t* kg = a.k + (size_t)group * a.Lmax * D;
        const __amdgpu_buffer_rsrc_t krs = make_rsrc(kg, n * D * 2);
        constexpr int NVO = C::CPR / C::RPI > 0 ? C::CPR / C::RPI : 1;
        int vo[NVO];
#pragma unroll
        for (int j = 0; j < NVO; ++j) {
            const int row = j * C::RPI + lane / C::CPR;
            vo[j] = (lane / C::CPR) * (D * 2) + (((lane % C::CPR) ^ (row % C::CPR)) * 16);
        }
        auto issue = [&](int key0, unsigned char* buf) {
#pragma unroll
            for (int i = 0; i < C::NLD; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    krs, (__attribute__((address_space(3))) void*)(buf + i * 1024), 16, vo[i % NVO],
                    (key0 + i * C::RPI) * (D * 2), 0, 0);
        };
        f32x4 sc[NT];
        if (wbase < n) issue(wbase, stage);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int key0 = wbase + t * C::KT;
            sc[t] = f32x4{NEG_INF, NEG_INF, NEG_INF, NEG_INF};
            if (key0 < n) {
                unsigned char* cur = stage + (t % C::NBUF) * C::STAGE_BYTES;
                const bool more = (t + 1 < NT) && (key0 + C::KT < n);
                if (C::NBUF == 2 && more) {
                    issue(key0 + C::KT, stage + ((t + 1) % C::NBUF) * C::STAGE_BYTES);
                    wait_vmem_n<C::NLD>();            // all but the next tile's loads have landed
                } else {
                    wait_vmem();                      // this tile's rows have landed in LDS
                }
                // two independent accumulators; the step loop is only partly
                // unrolled so that the LDS reads are not all hoisted into registers
                f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
                const unsigned char* srow = cur + ((mykey / C::RPI) * 64 + (mykey % C::RPI) * C::CPR) * 16;
                const int swz = mykey % C::CPR;
#pragma unroll 2
                for (int s = 0; s < C::STEPS; s += 2) {
                    const int c0 = s * C::BPT + cc, c1 = c0 + C::BPT;     // 16-byte chunks of the row
                    const u32x4 kb0 = *(const u32x4*)(srow + (c0 ^ swz) * 16);
                    const u32x4 qv0 = *(const u32x4*)&s_q[qrow_lds][c0 * 8];
                    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, qv0), __builtin_bit_cast(bf16x8, kb0), acc0, 0, 0, 0);
                    if (s + 1 < C::STEPS) {
                        const u32x4 kb1 = *(const u32x4*)(srow + (c1 ^ swz) * 16);
                        const u32x4 qv1 = *(const u32x4*)&s_q[qrow_lds][c1 * 8];
                        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, qv1), __builtin_bit_cast(bf16x8, kb1), acc1, 0, 0, 0);
                    }
                }
                const f32x4 acc = acc0 + acc1;
                wait_lds();                           // every read of the stage has returned
                if (C::NBUF == 1 && more) issue(key0 + C::KT, stage);
                const int key = key0 + mykey;
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
                for (int t = 0; t < NT; ++t) l += fast_exp2(sc[t][r] - m);
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
            // ---- exchange: publish (M, L), then merge every chunk's pair in
            // chunk order (this chunk's own from registers), so that all chunks
            // of the group reach the same LSE
            unsigned long long* ml = a.part_ml + (size_t)group * a.chunks * G + tid;   // chunk c: ml[c * G]
            const unsigned long long mine = ((unsigned long long)__float_as_uint(L) << 32) | __float_as_uint(M);
            if (a.chunks > 1)
                __hip_atomic_store(ml + (size_t)chunk * G, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            M = NEG_INF;
            L = 0.f;
            bool failed = false;
            for (int c0 = 0; c0 < a.chunks; c0 += 4) {        // four slots in flight (the scores hold most registers)
                unsigned long long v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int c = c0 + u;
                    v[u] = (c < a.chunks && c != chunk) ? load64(ml + (size_t)c * G) : mine;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (c0 + u < a.chunks) {
                        const unsigned long long x =
                            wait_slot64(ml + (size_t)(c0 + u) * G, v[u], spin_limit, a.status, failed);
                        const float m = __uint_as_float((unsigned)x), l = __uint_as_float((unsigned)(x >> 32));
                        if (l > 0.f) {
                            if (m > M) { L = L * exp2f(M - m) + l; M = m; }
                            else L += l * exp2f(m - M);
                        }
                    }
                }
            }
            if (failed) s_fail = 1;
            const float lse2 = M + __log2f(L);
            const int h = kv * G + tid;
            const float th = a.theta[(size_t)h * a.n_rows + min(n - 1, a.n_rows - 1)];
            // post-softmax: s >= theta; pre-softmax (kFlagPre): a >= theta
            s_T[tid] = (a.flags & kFlagPre) ? pre_log2_threshold(th) : log2_threshold(th, lse2);
            s_lse[tid] = lse2;
            s_M[tid] = M;
        }
        __syncthreads();

        // ---- phase 2: threshold, compaction, sparse V gather
        float Tr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool hv = hb + r < G;
            Tr[r] = hv ? s_T[hb + r] : INFINITY;
        }
        wait_lds();                            // no LDS read is left pending into the tile loop
        int ucount = 0;
        float acc[C::MFMA_ACC ? 1 : G][C::DPL];               // FMA path: [head][dims of this lane]
        f32x4 oacc[C::MFMA_ACC ? C::DB : 1];                   // MFMA path: O^T blocks (dims x heads)
        if constexpr (C::MFMA_ACC) {
#pragma unroll
            for (int db = 0; db < C::DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
        } else {
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int i = 0; i < C::DPL; ++i) acc[h][i] = 0.f;
        }

        const uint16_t* vg = a.v + (size_t)group * a.Lmax * D;
        const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vg, n * D * 2);

        // Kept keys (union over the group's heads) of all tiles of this wave are
        // listed in LDS with their per-head scores, which go to the wave's K
        // stage (phase 2 no longer needs it): the first CAPW entries there, any
        // further ones -- rows that keep nearly everything -- to the workspace
        // slot of the key.  Weights, kept counts and kept mass are then formed
        // once per listed entry, and the list is drained.
        float (*s_wl)[C::GW] = reinterpret_cast<float (*)[C::GW]>(stage);
        float* ovf = a.ovf_w + (size_t)group * a.Lmax * C::GW;
        int lcount = 0;
        const int keylane = lane - 16 * cc;      // lane that stands for this lane's key
        unsigned char* kmask = a.kept_mask ? a.kept_mask + ((size_t)b * a.Hq + (size_t)kv * G) * a.Lmax : nullptr;
        // the per-head kept mask, only where it is asked for
        // Tiles past the n valid keys hold -inf scores, which never reach a
        // threshold (thresholds are clamped to -FLT_MAX).  Bit t of kbits: some
        // head of the group keeps this lane's key of tile t (the lanes of one
        // key sit 16 lanes apart and are merged).  List slots follow the key
        // lanes in order, each lane's tiles in order: an exclusive prefix sum
        // of the per-lane counts, taken bit by bit with ballots.
        // A head keeps the key when x >= T, i.e. when x - T >= 0 (the rounded
        // difference of two floats has the sign of the exact one, and -inf - T
        // is -inf); the maximum over the lane's heads decides with one compare.
        unsigned kbits = 0u;
        if constexpr (!VOTE) {
            if (kmask) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const int key = wbase + t * C::KT + mykey;
                    if (key < n) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (hb + r < G) kmask[(size_t)(hb + r) * a.Lmax + key] = sc[t][r] >= Tr[r] ? 1 : 0;
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const float dmax = fmaxf(fmaxf(sc[t][0] - Tr[0], sc[t][1] - Tr[1]),
                                         fmaxf(sc[t][2] - Tr[2], sc[t][3] - Tr[3]));
                kbits |= (dmax >= 0.f) ? (1u << t) : 0u;
            }
            if (C::BPT >= 2) kbits |= __shfl_xor(kbits, 16);
            if (C::BPT == 4) kbits |= __shfl_xor(kbits, 32);
        } else {
            // GQA selection variants (Sec. 4.6): count, per key, the heads of
            // the group that keep it -- bit-sliced over the tiles (plane i holds
            // bit i of every tile's count), summed over the lanes that share the
            // key -- and load the key when the count reaches min_votes
            unsigned pl[5] = {0u, 0u, 0u, 0u, 0u};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                unsigned hm = 0u;
#pragma unroll
                for (int t = 0; t < NT; ++t) hm |= (sc[t][r] - Tr[r] >= 0.f) ? (1u << t) : 0u;
                votes_add(pl, hm);
            }
            if (C::BPT >= 2) votes_merge(pl, 16);
            if (C::BPT == 4) votes_merge(pl, 32);
            kbits = votes_at_least(pl, a.min_votes < 1 ? 1 : a.min_votes);
            if (kmask) {
                // per head: loaded, and kept by the head itself unless every
                // head uses all loaded keys
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const int key = wbase + t * C::KT + mykey;
                    if (key < n) {
                        const bool ld = (kbits >> t) & 1u;
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (hb + r < G)
                                kmask[(size_t)(hb + r) * a.Lmax + key] =
                                    (ld && (a.augment || sc[t][r] >= Tr[r])) ? 1 : 0;
                    }
                }
            }
        }
        const int kc = cc == 0 ? __popc(kbits) : 0;
        int lbase = 0, ltotal = 0;
#pragma unroll
        for (int bit = 0; (1 << bit) <= NT; ++bit) {
            const unsigned long long bb = __ballot((kc >> bit) & 1);
            lbase += (int)__builtin_amdgcn_mbcnt_hi((unsigned)(bb >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((unsigned)bb, 0u)) << bit;
            ltotal += __popcll(bb) << bit;
        }
        lbase = __shfl(lbase, keylane);
        {
            // Weights of the first CAPW entries go to the LDS list, later ones
            // (rows that keep nearly everything) to the workspace slot of their
            // key.  Lanes with nothing to store write spare slots of their own,
            // so the stores need no branch.
            const bool fits = ltotal <= C::CAPW;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const bool kept = (kbits >> t) & 1u;
                const int idx = lbase + __popc(kbits & ((1u << t) - 1u));
                const float4 wv = make_float4(sc[t][0], sc[t][1], sc[t][2], sc[t][3]);
                *(float4*)&s_wl[(kept && idx < C::CAPW) ? idx : C::SPARE + lane][hb] = wv;
                s_kl[wave][kept ? idx : C::WKEYS + lane] = (unsigned short)(t * C::KT + mykey);
                if (!fits) {
                    if (kept && idx >= C::CAPW) {
                        float* dst = &ovf[(size_t)(wbase + t * C::KT + mykey) * C::GW + hb];
                        publish(dst, wv.x); publish(dst + 1, wv.y); publish(dst + 2, wv.z); publish(dst + 3, wv.w);
                    }
                }
            }
            lcount = ltotal;
            // other lanes of this wave read the overflow weights back below:
            // the stores must have completed first (fits is wave-uniform)
            if (!fits) {
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                wait_vmem();
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
            }
        }
        ucount = lcount;
        wait_lds();
        // weights of the listed entries, one entry per lane: exact SDC keeps the
        // full softmax denominator, so the weight of a kept (key, head) is s
        float kmass_h[G];
        int kcnt_h[G];
#pragma unroll
        for (int h = 0; h < G; ++h) { kmass_h[h] = 0.f; kcnt_h[h] = 0; }
        {
            const int nl = lcount < C::CAPW ? lcount : C::CAPW;
            for (int e = lane; e < lcount; e += 64) {
                float x[C::GW];
                float* src = e < nl ? &s_wl[e][0] : ovf + (size_t)(wbase + s_kl[wave][e]) * C::GW;
#pragma unroll
                for (int h = 0; h < C::GW; ++h) x[h] = e < nl ? src[h] : consume(src + h);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const bool kp = (VOTE && a.augment) || x[h] >= s_T[h];
                    x[h] = kp ? fast_exp2(x[h] - s_lse[h]) : 0.f;
                    kmass_h[h] += x[h];
                    kcnt_h[h] += kp ? 1 : 0;
                }
#pragma unroll
                for (int h = G; h < C::GW; ++h) x[h] = 0.f;
                if (e < nl) {
#pragma unroll
                    for (int q4 = 0; q4 < C::GW; q4 += 4)
                        *(float4*)&src[q4] = make_float4(x[q4], x[q4 + 1], x[q4 + 2], x[q4 + 3]);
                } else {
#pragma unroll
                    for (int h = 0; h < C::GW; ++h) publish(src + h, x[h]);
                }
            }
        }
        wait_lds();
        if constexpr (C::MFMA_ACC) {
            // O^T += V^T W over the listed rows, 32 per MFMA step: the kept V
            // rows are fetched with buffer_load ... lds into the part of the
            // stage above the weights (16-byte chunk c of batch row j in slot
            // c ^ (j % CPR)), the rows past the batch's end up to its 32-row step are zeroed, and V^T
            // fragments come out of LDS transpose reads (in each 16-lane group,
            // lane i receives column i % 4 of the 8-byte rows addressed by lanes
            // i / 4 + 4 e).  The k-slot j of lane group lq stands for row
            // 8 lq + j of the step in both operands.  Weights enter as a bf16
            // high part and remainder (two MFMAs), heads in the 16 columns.
            const int nl = lcount < C::CAPW ? lcount : C::CAPW;
            const int wbytes = (nl * C::GW * 4 + 1023) & ~1023;
            unsigned char* vbuf = stage + wbytes;
            const int vrows_cap = ((C::NBUF * C::STAGE_BYTES - wbytes) / (D * 2)) / 32 * 32;
            const int l16 = lane & 15, lq = lane >> 4;
            int tr_off[2];                                     // byte offsets of the transpose reads, db = 0
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int j = 8 * lq + 4 * hh + l16 / 4;       // row of the step (steps start at multiples of 32)
                const int c = (4 * (l16 % 4)) / 8;
                tr_off[hh] = j * (D * 2) + ((c ^ (j % C::CPR)) * 16) + ((l16 % 4) & 1) * 8;
            }
            for (int b0 = 0; b0 < lcount; b0 += vrows_cap) {
                const int nrows = lcount - b0 < vrows_cap ? lcount - b0 : vrows_cap;
                const int nrows32 = (nrows + 31) & ~31;
                for (int i = 0; i * C::RPI < nrows; ++i) {
                    const int j = i * C::RPI + lane / C::CPR;
                    const int e = b0 + j;
                    const int key = wbase + (e < lcount ? (int)s_kl[wave][e] : 0);
                    const int chunk = (lane % C::CPR) ^ (j % C::CPR);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        vrs, (__attribute__((address_space(3))) void*)(vbuf + i * 1024), 16,
                        key * (D * 2) + chunk * 16, 0, 0, 0);
                }
                {
                    const int zr0 = (nrows + C::RPI - 1) / C::RPI * C::RPI;   // rows past the loaded ones
                    const u32x4 z = {0u, 0u, 0u, 0u};
                    for (int t = lane; t < (nrows32 - zr0) * C::CPR; t += 64)
                        *(u32x4*)(vbuf + (zr0 + t / C::CPR) * (D * 2) + (t % C::CPR) * 16) = z;
                }
                wait_vmem();
                wait_lds();
                for (int j0 = 0; j0 < nrows32; j0 += 32) {
                    // weights of rows j0 + 8 lq .. + 7 for head l16 (0 past the list or the heads)
                    float w[8];
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) {
                        const int e = b0 + j0 + 8 * lq + jj;
                        float x = 0.f;
                        if (l16 < G && e < lcount)
                            x = e < nl ? s_wl[e][l16] : consume(ovf + (size_t)(wbase + s_kl[wave][e]) * C::GW + l16);
                        w[jj] = x;
                    }
                    u32x4 whi, wlo;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        unsigned hi, lo;
                        split_bf16x2_pair(w[2 * q], w[2 * q + 1], hi, lo);
                        whi[q] = hi; wlo[q] = lo;
                    }
                    const bf16x8 bw = __builtin_bit_cast(bf16x8, whi), bwl = __builtin_bit_cast(bf16x8, wlo);
                    const unsigned char* vb = vbuf + j0 * (D * 2);
#pragma unroll
                    for (int db = 0; db < C::DB; ++db) {
                        const int dboff = (2 * db) * 16;       // chunk 2 db + c: XOR on bits c does not use
                        const dec_i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) dec_i16x4*)(vb + (tr_off[0] ^ dboff)));
                        const dec_i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) dec_i16x4*)(vb + (tr_off[1] ^ dboff)));
                        typedef short i16x8 __attribute__((ext_vector_type(8)));
                        const i16x8 v8 = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
                        const bf16x8 va = __builtin_bit_cast(bf16x8, v8);
                        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, bw, oacc[db], 0, 0, 0);
                        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, bwl, oacc[db], 0, 0, 0);
                    }
                }
                wait_lds();                                   // rows consumed before the next batch
            }
        } else {
            // The kept V rows are fetched with buffer_load ... lds into the part
            // of the stage above the weights (one 1 KiB instruction per RPI rows,
            // all of a batch in flight at once), then accumulated from LDS.
            // Weights of entries [0, CAPW) are in LDS, later ones in the workspace.
            const int nl = lcount < C::CAPW ? lcount : C::CAPW;
            const int wbytes = (nl * C::GW * 4 + 1023) & ~1023;
            unsigned char* vbuf = stage + wbytes;
            const int vrows_cap = ((C::NBUF * C::STAGE_BYTES - wbytes) / (D * 2)) / C::RPI * C::RPI;
            const int vlds = (lane % C::LPR) * C::DPL * 2;            // this lane's bytes in a row
            for (int b0 = 0; b0 < lcount; b0 += vrows_cap) {
                const int nrows = lcount - b0 < vrows_cap ? lcount - b0 : vrows_cap;
                for (int i = 0; i * C::RPI < nrows; ++i) {
                    const int e = b0 + i * C::RPI + lane / C::CPR;
                    const int key = wbase + (e < lcount ? (int)s_kl[wave][e] : 0);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        vrs, (__attribute__((address_space(3))) void*)(vbuf + i * 1024), 16,
                        key * (D * 2) + (lane % C::CPR) * 16, 0, 0, 0);
                }
                wait_vmem();
                for (int j = lane / C::LPR; j < nrows; j += C::RPG) {
                    const int e = b0 + j;
                    const typename VVec<C::DPL>::T raw =
                        *(const typename VVec<C::DPL>::T*)(vbuf + j * (D * 2) + vlds);
                    float vf[C::DPL];
                    unpack_bf16(raw, vf);
                    float wh[C::GW];
                    if (e < nl) {
#pragma unroll
                        for (int q4 = 0; q4 < C::GW; q4 += 4) {
                            const float4 x = *(const float4*)&s_wl[e][q4];
                            wh[q4] = x.x; wh[q4 + 1] = x.y; wh[q4 + 2] = x.z; wh[q4 + 3] = x.w;
                        }
                    } else {
                        const float* src = ovf + (size_t)(wbase + s_kl[wave][e]) * C::GW;
#pragma unroll
                        for (int q = 0; q < C::GW; ++q) wh[q] = consume(src + q);
                    }
#pragma unroll
                    for (int h = 0; h < G; ++h)
#pragma unroll
                        for (int i = 0; i < C::DPL; ++i) acc[h][i] = fmaf(wh[h], vf[i], acc[h][i]);
                }
                wait_lds();                                   // rows consumed before the next batch
            }
        }

        // ---- partial results of this workgroup
        if constexpr (C::MFMA_ACC) {
            __syncthreads();                   // every wave is done with its K staging
            // lane holds O^T[16 db + 4 lq + r][head l16]
            const int l16 = lane & 15, lq = lane >> 4;
            if (l16 < G) {
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int r = 0; r < 4; ++r) s_red[wave][l16][16 * db + 4 * lq + r] = oacc[db][r];
            }
        } else {
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int i = 0; i < C::DPL; ++i) {
                    float x = acc[h][i];
                    if (C::LPR == 16) x += __shfl_xor(x, 16);
                    x += __shfl_xor(x, 32);
                    acc[h][i] = x;
                }
            __syncthreads();                   // every wave is done with its K staging
            if (lane < C::LPR) {
#pragma unroll
                for (int h = 0; h < G; ++h)
#pragma unroll
                    for (int i = 0; i < C::DPL; ++i) s_red[wave][h][lane * C::DPL + i] = acc[h][i];
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float m = wave_sum(kmass_h[h]);
            const int c = wave_sum_i(kcnt_h[h]);
            if (lane == 0) { s_cm[wave][h] = m; s_cc[wave][h] = c; }
        }
        if (lane == 0) s_un[wave] = ucount;
        __syncthreads();
        const size_t pbase = (size_t)group * a.chunks + chunk;
        if (chunk > 0) {
            // ---- chunks 1..: publish the partials for chunk 0
            for (int idx = tid; idx < G * D; idx += C::THREADS) {
                float x = 0.f;
#pragma unroll
                for (int w = 0; w < C::WAVES; ++w) x += (&s_red[w][0][0])[idx];
                publish(a.part_out + pbase * G * D + idx, x);
            }
            if (tid < G) {
                float m = 0.f; int c = 0;
                for (int w = 0; w < C::WAVES; ++w) { m += s_cm[w][tid]; c += s_cc[w][tid]; }
                publish(a.part_mass + pbase * G + tid, m);
                publish_i(a.part_cnt + pbase * G + tid, c);
            }
            if (tid == 0) {
                int u = 0;
                for (int w = 0; w < C::WAVES; ++w) u += s_un[w];
                publish_i(a.part_union + pbase, s_fail ? -1 - u : u);
            }
        } else {
            // ---- chunk 0 combines, adding the partials in chunk order
            const bool renorm = (a.flags & 2u) != 0;
            const bool vmc = (a.flags & 1u) != 0 && !renorm;
            const size_t g0 = (size_t)group * a.chunks;
            bool failed = false;
            if (tid < G) {
                float m = 0.f; int c = 0;
                for (int w = 0; w < C::WAVES; ++w) { m += s_cm[w][tid]; c += s_cc[w][tid]; }
                m = gather_chunks(a.part_mass + g0 * G + tid, G, a.chunks, m, spin_limit, a.status, failed);
                c = gather_chunks(a.part_cnt + g0 * G + tid, G, a.chunks, c, spin_limit, a.status, failed);
                // Eq. 4 scale of the kept softmax values and the Eq. 6 beta; the
                // pre-softmax estimates of E~ relative to the full denominator:
                // exp-threshold gamma (n - k~) e^(theta - lse), offline E~ e^(max - lse)
                const int hq = kv * G + tid;
                const int rowid = min(n - 1, a.n_rows - 1);
                float etn = 0.f;
                if (a.flags & kFlagExpth)
                    etn = a.gamma * (float)(n - c) *
                          exp2f(a.theta[(size_t)hq * a.n_rows + rowid] * kLog2e - s_lse[tid]);
                if (a.flags & kFlagOffline)
                    etn = a.e_tilde[(size_t)hq * a.n_rows + rowid] * exp2f(s_M[tid] - s_lse[tid]);
                float fsc, bta;
                sdc_scale(a.flags, m, c, etn, fsc, bta);
                s_cm[0][tid] = m;
                s_cc[0][tid] = c;
                s_T[tid] = fsc;                // the threshold is no longer needed
                s_M[tid] = bta;
                const size_t o = (size_t)b * a.Hq + (size_t)kv * G + tid;
                if (a.kept_count) a.kept_count[o] = c;
                if (a.beta) a.beta[o] = bta;
                // every chunk has passed the exchange (it published after it):
                // its slots are empty again for the next call
                if (a.chunks > 1)
                    for (int ch = 0; ch < a.chunks; ++ch)
                        __hip_atomic_store(a.part_ml + (g0 + ch) * G + tid, kSlot64Empty, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
            }
            if (tid == 0) {
                int u = 0;
                for (int w = 0; w < C::WAVES; ++w) u += s_un[w];
                u = gather_union(a.part_union + g0, a.chunks, u, spin_limit, a.status, failed);
                if (a.vrows_read) a.vrows_read[group] = u;
            }
            if (failed) s_fail = 1;
            // running mean of V (Sec. 3.2.2, kept during generation): rows
            // 0..n-2 had mean mu; with row n-1 appended it is
            // ((n-1) mu + V[n-1]) / n, formed in float64 like the stand-alone update
            float* const mu_rw = a.v_mean_append;
            if (mu_rw != nullptr)
                for (int dd = tid; dd < D; dd += C::THREADS) {
                    const double prev = n > 1 ? (double)(n - 1) * (double)mu_rw[(size_t)group * D + dd] : 0.0;
                    const double vn = (double)bf16_bits_to_f32(a.v[((size_t)group * a.Lmax + (n - 1)) * D + dd]);
                    s_mu[dd] = (float)((prev + vn) / (double)n);
                }
            __syncthreads();
            for (int idx = tid; idx < G * D; idx += C::THREADS) {
                const int h = idx / D, dd = idx % D;
                float x = 0.f;
#pragma unroll
                for (int w = 0; w < C::WAVES; ++w) x += (&s_red[w][0][0])[idx];
                x = gather_chunks(a.part_out + g0 * G * D + idx, (size_t)G * D, a.chunks, x, spin_limit, a.status,
                                  failed);
                const float mass = s_cm[0][h];
                if (renorm) x = (s_cc[0][h] > 0) ? x / mass : 0.f;
                else if (a.flags & (kFlagExpth | kFlagOffline)) x *= s_T[h];
                if (vmc) x = fmaf(s_M[h], mu_rw != nullptr ? s_mu[dd] : a.v_mean[(size_t)group * D + dd], x);
                const size_t oi = ((size_t)b * a.Hq + (size_t)kv * G + h) * D + dd;
                if (a.flags & kFlagOutF32) ((float*)a.out)[oi] = x;
                else a.out[oi] = f32_to_bf16_bits(x);
            }
            // every read of the previous mean happened before the barrier above
            if (mu_rw != nullptr)
                for (int dd = tid; dd < D; dd += C::THREADS) mu_rw[(size_t)group * D + dd] = s_mu[dd];
            if (failed) s_fail = 1;
        }
        __syncthreads();
        // a wait of this group gave up (here, or in a chunk that flagged its
        // union): its outputs are poisoned rather than left as partial sums
        if (chunk == 0 && s_fail) poison_group<D, G>(a, b, kv, group, tid, C::THREADS);
    }
#endif
}

// Workspace of topth_decode_noalloc (for callers that cannot allocate): a
// static device array, one copy per GPU, large enough for the long-context
// shapes (batch 8 x 8 KV heads x 32768 keys at group size 8 needs 68 MiB).
constexpr size_t kScratchBytes = kNoallocScratchBytes;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// ------------------------------------------------------------------ host side
}  // namespace topth

#include <atomic>
#include <mutex>

namespace topth {

namespace {

struct Variant {
    int (*launch)(int grid, hipStream_t stream, const DecodeKArgs& a);
    int (*resident)(int* per_cu);
    int keys_per_wg;
};

// Register tiles per wave offered for each group size: the largest ones are
// left out where the scores would no longer fit in registers at two waves per
// SIMD without spilling.
constexpr int kMaxVariants = 4;

template <int D, int G, int NT, bool VOTE>
int launch_variant(int grid, hipStream_t stream, const DecodeKArgs& a) {
    hipLaunchKernelGGL((decode_bf16_kernel<D, G, NT, VOTE>), dim3(grid), dim3(kDecodeWaves * 64), 0, stream, a);
    return hipGetLastError();
}

template <int D, int G, int NT, bool VOTE>
int resident_variant(int* per_cu) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, (const void*)decode_bf16_kernel<D, G, NT, VOTE>,
                                                        kDecodeWaves * 64, 0);
}

template <int D, int G, int NT, bool VOTE>
Variant make_variant() {
    return {launch_variant<D, G, NT, VOTE>, resident_variant<D, G, NT, VOTE>, DecodeCfg<D, G, NT>::KEYS_PER_WG};
}

// The vote variants leave out 32 tiles per wave: the vote count's registers
// next to 32 score tiles would spill.
template <int D, int G, bool VOTE>
int variants_for(Variant* out) {
    int k = 0;
    out[k++] = make_variant<D, G, 4, VOTE>();
    out[k++] = make_variant<D, G, 8, VOTE>();
    if constexpr (G != 16) out[k++] = make_variant<D, G, 16, VOTE>();
    if constexpr (G == 8 && !VOTE) out[k++] = make_variant<D, G, 32, VOTE>();   // one head: its K list would not fit in LDS
    return k;
}

template <bool VOTE>
int variants(int d, int G, Variant* out) {
    if (d == 64) {
        switch (G) {
            case 1: return variants_for<64, 1, VOTE>(out);
            case 2: return variants_for<64, 2, VOTE>(out);
            case 4: return variants_for<64, 4, VOTE>(out);
            case 8: return variants_for<64, 8, VOTE>(out);
            default: return variants_for<64, 16, VOTE>(out);
        }
    }
    switch (G) {
        case 1: return variants_for<128, 1, VOTE>(out);
        case 2: return variants_for<128, 2, VOTE>(out);
        case 4: return variants_for<128, 4, VOTE>(out);
        case 8: return variants_for<128, 8, VOTE>(out);
        default: return variants_for<128, 16, VOTE>(out);
    }
}

int keys_per_wg_min(int G) {
    const int P = (G <= 4) ? 4 : (G == 8 ? 2 : 1);
    return 4 * 4 * 16 * P;
}

// Resident workgroups per CU of each kernel variant and the CU count, per
// device, computed once (the occupancy query is slow next to a decode step).
// Entries are atomics: concurrent first calls may both run the query, and
// both store the same value.
struct DeviceInfo {
    std::atomic<int> cus{0};
    std::atomic<int> occ[2][2][17][kMaxVariants] = {};   // [vote][d==128][G][variant] -> workgroups per CU (0 = unknown)
};
DeviceInfo g_dev[16];

int resident_per_cu(int dev, bool vote, int d, int G, int vi, const Variant& v, int* out) {
    std::atomic<int>& slot = g_dev[dev].occ[vote][d == 128][G][vi];
    int val = slot.load(std::memory_order_relaxed);
    if (val == 0) {
        int per_cu = 0;
        const int e = v.resident(&per_cu);
        if (e != hipSuccess) return e;
        val = per_cu > 0 ? per_cu : -1;
        slot.store(val, std::memory_order_relaxed);
    }
    *out = val > 0 ? val : 0;
    return hipSuccess;
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
    bytes += pc * G * sizeof(unsigned long long);
    bytes += pc * G * d * sizeof(float);
    bytes += pc * G * sizeof(float);
    bytes += pc * G * sizeof(int);
    bytes += pc * sizeof(int);
    bytes += groups * (size_t)Lmax * (G < 4 ? 4 : G) * sizeof(float);   // weight overflow slots
    return bytes + 1024;
}

// Launch plan of one decode call: the kernel variant, the grid and where the
// exchange slots and overflow weights sit in the workspace.
struct DecodePlan {
    Variant v;
    int chunks, items, grid;
    size_t off_ml, off_out, off_mass, off_cnt, off_union, off_ovf;
    size_t slots_end;      // end of the header and exchange slots (the part that must be prepared)
    size_t ws_end;         // bytes of workspace the call uses
};

int plan_decode_bf16(const DecodeParams& p, DecodePlan* plan) {
    const int G = p.Hq / p.Hkv;
    const int groups = p.B * p.Hkv;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 16) return hipErrorInvalidDevice;
    int cus = g_dev[dev].cus.load(std::memory_order_relaxed);
    if (cus == 0) {
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        g_dev[dev].cus.store(cus, std::memory_order_relaxed);
    }

    // The smallest register footprint whose work fits in one resident round;
    // otherwise the largest (fewest rounds).  Every workgroup of the grid is
    // resident at once (grid <= resident capacity), so the chunks of a group
    // that wait for each other in the exchange always run concurrently.
    Variant vs[kMaxVariants];
    const bool vote = p.min_votes > 1 || p.augment;
    const int nv = vote ? variants<true>(p.d, G, vs) : variants<false>(p.d, G, vs);
    Variant v{};
    int chunks = 0, capacity = 0;
    for (int vi = 0; vi < nv; ++vi) {
        int per_cu = 0;
        e = (hipError_t)resident_per_cu(dev, vote, p.d, G, vi, vs[vi], &per_cu);
        if (e != hipSuccess) return e;
        v = vs[vi];
        capacity = per_cu * cus;
        chunks = (p.Lmax + v.keys_per_wg - 1) / v.keys_per_wg;
        if ((long long)chunks * groups <= capacity) break;
    }
    if (capacity <= 0 || chunks > capacity) return hipErrorInvalidConfiguration;
    plan->v = v;
    plan->chunks = chunks;
    plan->items = chunks * groups;
    plan->grid = std::min(plan->items, (capacity / chunks) * chunks);

    // workspace carve-up (the header holds the status word and the spin limit)
    const size_t pc = (size_t)plan->items;
    size_t off = kWsHeaderBytes;
    plan->off_ml = off; off += pc * G * sizeof(unsigned long long);
    plan->off_out = off; off += pc * G * p.d * sizeof(float);
    plan->off_mass = off; off += pc * G * sizeof(float);
    plan->off_cnt = off; off += pc * G * sizeof(int);
    plan->off_union = off; off += pc * sizeof(int);
    plan->slots_end = off;
    off = (off + 255) & ~(size_t)255;
    plan->off_ovf = off; off += (size_t)groups * p.Lmax * (G < 4 ? 4 : G) * sizeof(float);
    plan->ws_end = off;
    return hipSuccess;
}

int launch_decode_bf16_planned(const DecodeParams& p, const DecodePlan& plan, bool prepare, hipStream_t stream) {
    if (plan.ws_end > p.ws_bytes) return hipErrorInvalidValue;
    char* ws = (char*)p.ws;
    if (prepare) {
        // header zero, exchange slots empty: what a prepared workspace holds
        int e = launch_ws_prepare(ws, kWsHeaderBytes, plan.slots_end, stream);
        if (e != hipSuccess) return e;
    }
    DecodeKArgs a = {};
    a.q = (const uint16_t*)p.q; a.k = (const uint16_t*)p.k; a.v = (const uint16_t*)p.v;
    a.seq_lens = p.seq_lens; a.theta = p.theta; a.v_mean = p.v_mean; a.v_mean_append = p.v_mean_append;
    a.e_tilde = p.e_tilde; a.gamma = p.gamma;
    a.min_votes = p.min_votes; a.augment = p.augment;
    a.out = (uint16_t*)p.out; a.kept_count = p.kept_count; a.beta = p.beta; a.vrows_read = p.vrows_read;
    a.kept_mask = p.kept_mask;
    a.status = (int*)ws;
    a.part_ml = (unsigned long long*)(ws + plan.off_ml);
    a.part_out = (float*)(ws + plan.off_out);
    a.part_mass = (float*)(ws + plan.off_mass);
    a.part_cnt = (int*)(ws + plan.off_cnt);
    a.part_union = (int*)(ws + plan.off_union);
    a.ovf_w = (float*)(ws + plan.off_ovf);
    a.B = p.B; a.Hq = p.Hq; a.Hkv = p.Hkv; a.Lmax = p.Lmax; a.n_rows = p.n_rows;
    a.chunks = plan.chunks; a.items = plan.items;
    a.xscale = p.scale * kLog2e;
    a.flags = p.flags;
    a.xcd_map = (plan.grid % (8 * plan.chunks) == 0 && plan.items % plan.grid == 0) ? 1 : 0;
    return plan.v.launch(plan.grid, stream, a);
}

int launch_decode_bf16(const DecodeParams& p, hipStream_t stream) {
    DecodePlan plan;
    const int e = plan_decode_bf16(p, &plan);
    if (e != hipSuccess) return e;
    return launch_decode_bf16_planned(p, plan, false, stream);
}

// ------------------------------------------------------------ no-allocation
// topth_decode_noalloc takes its workspace from `scratch`, one copy per GPU
// (held until the process ends).  In host code the array's name is only a
// stand-in: its device address on the current GPU comes from
// hipGetSymbolAddress, once per device, and only that address is used.
std::mutex g_scratch_mu;
void* g_scratch_addr[16] = {};

int scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 16) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_addr[dev] == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (ptr == nullptr) return hipErrorInvalidSymbol;
        g_scratch_addr[dev] = ptr;
    }
    *out = g_scratch_addr[dev];
    return hipSuccess;
}

size_t noalloc_scratch_bytes() { return kScratchBytes; }

// Plans the call, checks that it fits the scratch (*fits = false otherwise,
// nothing enqueued), then prepares the header and slots of this call's layout
// and launches.  Every call prepares them anew, so a call whose exchange gave
// up leaves nothing that a later call reads.
int launch_decode_bf16_noalloc(DecodeParams p, bool* fits, hipStream_t stream) {
    DecodePlan plan;
    int e = plan_decode_bf16(p, &plan);
    if (e != hipSuccess) return e;
    *fits = plan.ws_end <= kScratchBytes;
    if (!*fits) return hipSuccess;
    e = scratch_address(&p.ws);
    if (e != hipSuccess) return e;
    p.ws_bytes = kScratchBytes;
    return launch_decode_bf16_planned(p, plan, true, stream);
}

int noalloc_scratch(void** out) { return scratch_address(out); }

}  // namespace topth
