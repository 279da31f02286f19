// Device half of libgrpo for gfx950 (CDNA4): the fused token-level GRPO loss
// forward/backward, the forward-only log-prob pass, the row/chunk statistics
// reductions, and two small layout helpers.
//
// Sources: [P1] "Sizing mini-batches and micro-batches" ("The hard part:
// deferred normalization", "pi_old must be frozen across the window");
// [P2] "03 Data Protocol and Batch Lifecycle" ("Field Lineage": response
// mask, advantage broadcast); [P4] "How a context-compaction step fits a
// variable number of rows into one batch" ("Why the row count does not change
// the math").
//
// Design (HBM-bound streaming, no MFMA: there is no contraction here).
// The fused loss reads a token's row of V logits from HBM once and keeps it
// on chip until its gradient row is written (tok_reg_kernel):
//   * large V (e.g. 151936 bf16 = 297 KiB): one 1024-thread workgroup per
//     token; each lane holds NV 16-byte vectors (NV = 19 -> 76 VGPRs), and
//     past that 9 more per lane in LDS (rows up to 229376 bf16).  bf16 rows up
//     to 262144 read the up to 4 vectors per lane past that in both sweeps.
//     Reductions: wave64 butterfly, then the 16 wave partials through LDS in a
//     fixed order.
//   * small V (<= 4096 bf16 / 2048 fp32): one wave64 per token, four tokens
//     per 256-thread workgroup, no LDS and no barrier at all.
// One sweep over the row forms sum 2^t and sum 2^t * t with a per-lane shift
// (t = z*log2(e) - c) and merges the lanes exactly; a second writes
// dz = coef * 2^(z*log2(e) - lse*log2(e)) minus coef at the target.  So the
// kernel moves V*(in + out) bytes per valid token and V*out per masked one.
// Rows off 16-byte alignment, or past what registers and LDS hold, take
// tok_stream_kernel: 256 threads per token, the row streamed once for the sums
// and once more for dz.  The forward-only pass keeps no row on chip: rows past
// 1024 vectors take tok_stream_kernel's single sum sweep, shorter ones
// tok_reg_kernel.
//
// Every reduction has a fixed order, nothing uses floating-point atomics, so
// results are bit-for-bit reproducible and a token's outputs depend only on
// its own row, never on its position in the chunk.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "common.h"
#include "surrogate.h"

using grpo::fail;
using grpo::ok;

namespace {

using grpo_dev::kLn2;
using grpo_dev::kLog2e;
constexpr float kNegClampLog2 = -128.0f;   // below this 2^t is under every fp32 normal

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    bf16x2 r = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

// The same for -lo and -hi, the negation taken by the instruction's source
// modifiers (no separate sign flip).
__device__ __forceinline__ uint32_t pack_bf16x2_neg(float lo, float hi) {
    uint32_t r;
    asm("v_cvt_pk_bf16_f32 %0, -%1, -%2" : "=v"(r) : "v"(lo), "v"(hi));
    return r;
}

// ---------------------------------------------------------------- dtype traits

template <int DT> struct In;
template <> struct In<GRPO_BF16> {
    static constexpr int VEC = 8;                      // elements per 16-byte vector
    static constexpr int BYTES = 2;
    static constexpr uint32_t NEG_INF2 = 0xff80ff80u;  // two bf16 -inf
    __device__ static __forceinline__ void unpack(const uint4& v, float (&f)[8]) {
        f[0] = bf_lo(v.x); f[1] = bf_hi(v.x); f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
        f[4] = bf_lo(v.z); f[5] = bf_hi(v.z); f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
    }
    __device__ static __forceinline__ float scalar(const void* row, int64_t i) {
        const uint16_t b = reinterpret_cast<const uint16_t*>(row)[i];
        return __uint_as_float((uint32_t)b << 16);
    }
};
template <> struct In<GRPO_F32> {
    static constexpr int VEC = 4;
    static constexpr int BYTES = 4;
    static constexpr uint32_t NEG_INF2 = 0xff800000u;  // one fp32 -inf
    __device__ static __forceinline__ void unpack(const uint4& v, float (&f)[4]) {
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    }
    __device__ static __forceinline__ float scalar(const void* row, int64_t i) {
        return reinterpret_cast<const float*>(row)[i];
    }
};

// 16- or 8-byte global stores.  st16 is the plain store, used for the
// gradient rows of valid tokens (read and written in the same sweep).
// st16_nt is the non-temporal form, used for the zero rows of masked tokens:
// a write-only stream that is never read back by this kernel.  (Measured:
// non-temporal zero rows are ~3 % faster on a batch that is half padding;
// non-temporal stores for the valid rows are ~7 % slower on a batch without
// padding.)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <typename T>
__device__ __forceinline__ void st16(T* p, const T& v) {
    *p = v;
}
template <typename T>
__device__ __forceinline__ void st16_nt(T* p, const T& v) {
    if constexpr (sizeof(T) == 16) __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(p));
    else __builtin_nontemporal_store(__builtin_bit_cast(u32x2, v), reinterpret_cast<u32x2*>(p));
}

template <int DT> struct Out;
template <> struct Out<GRPO_BF16> {
    static constexpr int BYTES = 2;
    // neg: every stored value negated (sign bits flipped after rounding)
    template <int N>
    __device__ static __forceinline__ void store(void* row, int64_t e0, const float (&d)[N], bool neg = false) {
        uint16_t* p = reinterpret_cast<uint16_t*>(row) + e0;
        const uint32_t sg = neg ? 0x80008000u : 0u;
        if constexpr (N == 8) {
            uint4 v;
            if (neg) {   // (uniform per token) the sign rides on the conversion
                v.x = pack_bf16x2_neg(d[0], d[1]); v.y = pack_bf16x2_neg(d[2], d[3]);
                v.z = pack_bf16x2_neg(d[4], d[5]); v.w = pack_bf16x2_neg(d[6], d[7]);
            } else {
                v.x = pack_bf16x2(d[0], d[1]); v.y = pack_bf16x2(d[2], d[3]);
                v.z = pack_bf16x2(d[4], d[5]); v.w = pack_bf16x2(d[6], d[7]);
            }
            st16(reinterpret_cast<uint4*>(p), v);
        } else {
            uint2 v;
            v.x = pack_bf16x2(d[0], d[1]) ^ sg; v.y = pack_bf16x2(d[2], d[3]) ^ sg;
            st16(reinterpret_cast<uint2*>(p), v);
        }
    }
    template <int N>
    __device__ static __forceinline__ void zero(void* row, int64_t e0) {
        uint16_t* p = reinterpret_cast<uint16_t*>(row) + e0;
        if constexpr (N == 8) st16_nt(reinterpret_cast<uint4*>(p), make_uint4(0, 0, 0, 0));
        else st16_nt(reinterpret_cast<uint2*>(p), make_uint2(0, 0));
    }
    __device__ static __forceinline__ void scalar(void* row, int64_t i, float d) {
        f32x2 v = {d, 0.0f};
        bf16x2 r = __builtin_convertvector(v, bf16x2);
        reinterpret_cast<uint16_t*>(row)[i] = (uint16_t)(__builtin_bit_cast(uint32_t, r) & 0xffffu);
    }
};
template <> struct Out<GRPO_F32> {
    static constexpr int BYTES = 4;
    template <int N>
    __device__ static __forceinline__ void store(void* row, int64_t e0, const float (&d)[N], bool neg = false) {
        uint4* p = reinterpret_cast<uint4*>(reinterpret_cast<float*>(row) + e0);
        const uint32_t sg = neg ? 0x80000000u : 0u;
        st16(p, make_uint4(__float_as_uint(d[0]) ^ sg, __float_as_uint(d[1]) ^ sg, __float_as_uint(d[2]) ^ sg,
                           __float_as_uint(d[3]) ^ sg));
        if constexpr (N == 8)
            st16(p + 1, make_uint4(__float_as_uint(d[4]) ^ sg, __float_as_uint(d[5]) ^ sg,
                                   __float_as_uint(d[6]) ^ sg, __float_as_uint(d[7]) ^ sg));
    }
    template <int N>
    __device__ static __forceinline__ void zero(void* row, int64_t e0) {
        float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(row) + e0);
        st16_nt(p, make_float4(0.f, 0.f, 0.f, 0.f));
        if constexpr (N == 8) st16_nt(p + 1, make_float4(0.f, 0.f, 0.f, 0.f));
    }
    __device__ static __forceinline__ void scalar(void* row, int64_t i, float d) {
        reinterpret_cast<float*>(row)[i] = d;
    }
};

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
// Butterfly: every lane ends with the same bits (each step adds the same pair).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}
__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}
__device__ __forceinline__ long long wave_sum_i(long long x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// (c, s, w) of two parts of a row merged exactly, where a part's s = sum 2^t
// and w = sum 2^t * t with t = z*log2(e) - c: relative to C = max(c, c2),
// s = s 2^(c-C) + s2 2^(c2-C) and w = sum over both of 2^(c_i-C) (w_i +
// (c_i-C) s_i).  An empty part (s = 0) leaves the other as it is.
__device__ __forceinline__ void merge3(float& c, float& s, float& w, float c2, float s2, float w2) {
    if (s2 == 0.0f) return;
    if (s == 0.0f) {
        c = c2;
        s = s2;
        w = w2;
        return;
    }
    const float C = fmaxf(c, c2);
    const float d1 = c - C, d2 = c2 - C;
    const float f1 = __builtin_amdgcn_exp2f(d1), f2 = __builtin_amdgcn_exp2f(d2);
    const float S = fmaf(s, f1, s2 * f2);
    w = fmaf(f1, fmaf(s, d1, w), f2 * fmaf(s2, d2, w2));
    s = S;
    c = C;
}

// Butterfly over the lanes of a wave with stride o >= 1 down to 1, starting
// at `from`: both lanes of a pair merge (lower lane's part, upper lane's
// part), so every lane ends with the same bits.
__device__ __forceinline__ void butterfly3(float& c, float& s, float& w, int lane, int from) {
#pragma unroll
    for (int o = from; o > 0; o >>= 1) {
        float c2 = __shfl_xor(c, o), s2 = __shfl_xor(s, o), w2 = __shfl_xor(w, o);
        if (lane & o) {
            const float tc = c, ts = s, tw = w;
            c = c2; s = s2; w = w2;
            c2 = tc; s2 = ts; w2 = tw;
        }
        merge3(c, s, w, c2, s2, w2);
    }
}

// The row's (c, s, w) on every thread of the TPR threads of a row: wave
// butterfly, then the WPR wave parts through LDS, merged by a butterfly over
// the first WPR lanes of every wave (the same fixed tree everywhere).
template <int WPR>
__device__ __forceinline__ void block_merge(float& c, float& s, float& w, int tid, float (*s_part)[3]) {
    const int lane = tid & 63;
    butterfly3(c, s, w, lane, 32);
    if constexpr (WPR > 1) {
        if (lane == 0) {
            s_part[tid >> 6][0] = c;
            s_part[tid >> 6][1] = s;
            s_part[tid >> 6][2] = w;
        }
        __syncthreads();
        c = -INFINITY;
        s = 0.0f;
        w = 0.0f;
        if (lane < WPR) {
            c = s_part[lane][0];
            s = s_part[lane][1];
            w = s_part[lane][2];
        }
        butterfly3(c, s, w, lane, WPR / 2);
        c = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(c)));
        s = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(s)));
        w = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(w)));
    }
}

// Row maximum and row sums on every thread (wave butterfly, then the wave
// parts through LDS in wave order); the LDS buffer may still be being read
// by an earlier helper, hence the leading barrier.
template <int WPR>
__device__ __forceinline__ float block_max(float m, int tid, float (*s_part)[3]) {
    m = wave_max(m);
    if constexpr (WPR > 1) {
        __syncthreads();
        if ((tid & 63) == 0) s_part[tid >> 6][0] = m;
        __syncthreads();
        m = s_part[0][0];
#pragma unroll
        for (int i = 1; i < WPR; ++i) m = fmaxf(m, s_part[i][0]);
    }
    return m;
}

template <int WPR>
__device__ __forceinline__ void block_sum2(float& s, float& w, int tid, float (*s_part)[3]) {
    s = wave_sum(s);
    w = wave_sum(w);
    if constexpr (WPR > 1) {
        __syncthreads();
        if ((tid & 63) == 0) {
            s_part[tid >> 6][1] = s;
            s_part[tid >> 6][2] = w;
        }
        __syncthreads();
        s = s_part[0][1];
        w = s_part[0][2];
#pragma unroll
        for (int i = 1; i < WPR; ++i) {
            s += s_part[i][1];
            w += s_part[i][2];
        }
    }
}

// An empty asm that claims to rewrite the register-resident row: the unpacked
// floats of one sweep cannot then be kept alive into the next sweep (that
// would double the row's register footprint and spill); each sweep re-derives
// them from the packed registers with one ALU op per element.
__device__ __forceinline__ void opaque_vec(uint4& x) {
    asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w));
}
template <int NV>
__device__ __forceinline__ void opaque_regs(uint4 (&x)[NV]) {
#pragma unroll
    for (int k = 0; k < NV; ++k) opaque_vec(x[k]);
}

// ---------------------------------------------------------------- parameters

struct TokParams {
    const void* logits;
    int64_t ld;
    int64_t n_tok;
    int64_t V;
    const int32_t* target;
    const uint8_t* mask;
    const float* old_logp;
    const int32_t* tok_row;
    const float* adv_row;
    int64_t n_rows;
    float eps_low, eps_high, scale;
    const int64_t* denom;
    void* dlogits;
    int64_t ld_out;
    float* logp;
    float* lse;
    float* entropy;
    float* loss_tok;
    uint8_t* tok_flags;
    grpo_dev::Terms terms;   // row weights, entropy bonus, KL
    float* kl_tok;           // required when terms.ref_logp is set
    const int64_t* tok_src;  // NULL, or the batch token row behind chunk token t
    int64_t n_src;
};

// Batch row of chunk token t (t itself without a source map); -1 when the
// map points outside the batch.
__device__ __forceinline__ int64_t token_source(const TokParams& p, int64_t t) {
    if (!p.tok_src) return t;
    const int64_t s = p.tok_src[t];
    return (uint64_t)s < (uint64_t)p.n_src ? s : -1;
}

// Per-token scalar tail shared by both kernels: from (max-shifted sums, z_y)
// to logp / entropy / surrogate / gradient coefficient.  c = the log2-domain
// shift used for the sums, s = sum 2^t, w = sum 2^t * t.
struct TokenResult {
    float c2;      // log2-domain logsumexp: p_v = 2^(z_v*log2e - c2)
    float coef;    // dlogits_v = p_v * (ea + eb * t_v) - coef * [v == y], t_v = z_v*log2e - c2
    float ea;      // coef + e*H
    float eb;      // e*ln2, e = ent_coef * s (0: dlogits_v = coef * (p_v - [v == y]))
};

template <bool GRAD>
__device__ __forceinline__ TokenResult token_tail(const TokParams& p, int64_t t, int64_t src, float c, float s,
                                                  float w, float zy, bool ybad, bool write) {
    const float log2s = log2f(s);
    const float c2 = c + log2s;
    const float lse = c2 * kLn2;
    const float logp = ybad ? __builtin_nanf("") : zy - lse;
    const float H = kLn2 * (log2s - w / s);
    TokenResult r{c2, 0.0f, 0.0f, 0.0f};
    if constexpr (!GRAD) {
        if (write) {
            p.logp[t] = logp;
            if (p.lse) p.lse[t] = lse;
            if (p.entropy) p.entropy[t] = H;
        }
        return r;
    } else {
        const int32_t row = p.tok_row[t];
        const float A = ((uint32_t)row < (uint64_t)p.n_rows) ? p.adv_row[row] : __builtin_nanf("");
        const float sf = grpo_dev::token_factor(grpo_dev::step_scale(p.scale, p.denom), p.terms.row_weight, row,
                                                p.n_rows);
        const grpo_dev::Surrogate sg = grpo_dev::surrogate(logp, H, p.old_logp[src], A, p.eps_low, p.eps_high, sf,
                                                           p.terms, src);
        if (write) {
            p.logp[t] = logp;
            if (p.lse) p.lse[t] = lse;
            p.entropy[t] = H;
            p.loss_tok[t] = sg.loss;
            if (p.kl_tok) p.kl_tok[t] = sg.kl;
            p.tok_flags[t] = (uint8_t)(1u | (sg.clipped ? 2u : 0u) | (sg.bad ? 4u : 0u));
        }
        r.coef = sg.coef;
        if (p.terms.ent_coef != 0.0f) {
            const float e = p.terms.ent_coef * sf;
            r.ea = fmaf(e, H, sg.coef);
            r.eb = e * kLn2;
        } else {
            r.ea = sg.coef;
        }
        return r;
    }
}

template <bool GRAD>
__device__ __forceinline__ void masked_outputs(const TokParams& p, int64_t t) {
    p.logp[t] = 0.0f;
    if (p.lse) p.lse[t] = 0.0f;
    if (p.entropy) p.entropy[t] = 0.0f;
    if constexpr (GRAD) {
        p.loss_tok[t] = 0.0f;
        if (p.kl_tok) p.kl_tok[t] = 0.0f;
        p.tok_flags[t] = 0;
    }
}

// A chunk token whose source index is outside the batch: nothing V-sized is
// touched; the token is reported valid and non-finite, which poisons the window.
template <bool GRAD>
__device__ __forceinline__ void bad_source_outputs(const TokParams& p, int64_t t) {
    p.logp[t] = __builtin_nanf("");
    if (p.lse) p.lse[t] = 0.0f;
    if (p.entropy) p.entropy[t] = 0.0f;
    if constexpr (GRAD) {
        p.loss_tok[t] = 0.0f;
        if (p.kl_tok) p.kl_tok[t] = 0.0f;
        p.tok_flags[t] = 1u | 4u;
    }
}

// dlogits value of one element with the entropy bonus on: p * (ea + eb * tt)
// with p = 2^tt (an element with p = 0 contributes 0, also at z = -inf)
__device__ __forceinline__ float dz_with_bonus(float tt, float ea, float eb) {
    const float pp = __builtin_amdgcn_exp2f(tt);
    return pp > 0.0f ? pp * fmaf(eb, tt, ea) : 0.0f;
}

// Block -> token group.  Hardware dispatch sends block b to XCD b % 8; the
// groups are dealt to the XCDs in runs of 16 consecutive groups instead of one
// by one, so that a mask pattern with a short period in token order (valid
// and masked tokens alternating, say) does not put all the valid tokens on
// half of the XCDs.  A bijection on [0, nb): blocks below the largest
// multiple of 8 x 16 are permuted, the rest map to themselves.
__device__ __forceinline__ uint32_t xcd_runs(uint32_t b, uint32_t nb) {
    constexpr uint32_t kXcd = 8, kRun = 16;
    const uint32_t full = nb / (kXcd * kRun) * (kXcd * kRun);
    if (b >= full) return b;
    const uint32_t x = b % kXcd, j = b / kXcd;
    return ((j / kRun) * kXcd + x) * kRun + j % kRun;
}

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate: at most n vector-memory operations of this wave still
// outstanding (vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt not waited on)
#define GRPO_LOSS_VMCNT(n) (((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

// Per-vector steps of the sweeps, shared by the register-resident vectors and
// the ones held in LDS.
template <int DTI>
__device__ __forceinline__ void sweep_sums(const uint4& v, float c, float& s, float& w) {
    constexpr int VEC = In<DTI>::VEC;
    float f[VEC];
    In<DTI>::unpack(v, f);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        const float tt = fmaf(f[e], kLog2e, -c);
        const float ee = __builtin_amdgcn_exp2f(tt);
        s += ee;
        w = fmaf(ee, tt, w);
    }
}

template <int DTI>
__device__ __forceinline__ void sweep_max(const uint4& v, float& m) {
    constexpr int VEC = In<DTI>::VEC;
    float f[VEC];
    In<DTI>::unpack(v, f);
#pragma unroll
    for (int e = 0; e < VEC; ++e) m = fmaxf(m, f[e]);
}

template <int DTI>
__device__ __forceinline__ void sweep_sums_clamped(const uint4& v, float c, float& s, float& w) {
    constexpr int VEC = In<DTI>::VEC;
    float f[VEC];
    In<DTI>::unpack(v, f);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        const float tt = fmaf(f[e], kLog2e, -c);
        const float ee = __builtin_amdgcn_exp2f(tt);
        s += ee;
        w = fmaf(ee, fmaxf(tt, kNegClampLog2), w);
    }
}

// Rows off 16-byte alignment (register kernel, MIS): the row is read through
// the aligned vectors that cover it, and the first and last of those hold
// elements outside the row.  For such a vector, elements e with
// elo <= e < ehi belong to the row (element e of vector idx is row element
// idx*VEC + e - hb); these helpers take only those.
template <int DTI>
__device__ __forceinline__ void sweep_sums_part(const uint4& v, int elo, int ehi, float c, float& s, float& w,
                                                bool clamp) {
    constexpr int VEC = In<DTI>::VEC;
    float f[VEC];
    In<DTI>::unpack(v, f);
#pragma unroll
    for (int e = 0; e < VEC; ++e)
        if (e >= elo && e < ehi) {
            const float tt = fmaf(f[e], kLog2e, -c);
            const float ee = __builtin_amdgcn_exp2f(tt);
            s += ee;
            w = fmaf(ee, clamp ? fmaxf(tt, kNegClampLog2) : tt, w);
        }
}

template <int DTI>
__device__ __forceinline__ void sweep_max_part(const uint4& v, int elo, int ehi, float& m) {
    constexpr int VEC = In<DTI>::VEC;
    float f[VEC];
    In<DTI>::unpack(v, f);
#pragma unroll
    for (int e = 0; e < VEC; ++e)
        if (e >= elo && e < ehi) m = fmaxf(m, f[e]);
}

// dz of the row's elements in a partial vector, stored one element at a time
// (the vector's other elements belong to neighbouring rows: never written)
template <int DTI, int DTO>
__device__ __forceinline__ void dz_part(void* orow, int64_t e0, const uint4& v, const TokenResult& r, float c3,
                                        bool neg, int elo, int ehi) {
    constexpr int VEC = In<DTI>::VEC;
    float f[VEC];
    In<DTI>::unpack(v, f);
#pragma unroll
    for (int e = 0; e < VEC; ++e)
        if (e >= elo && e < ehi) {
            float d;
            if (r.eb == 0.0f) {
                d = __builtin_amdgcn_exp2f(fmaf(f[e], kLog2e, -c3));
                d = neg ? -d : d;
            } else {
                d = dz_with_bonus(fmaf(f[e], kLog2e, -r.c2), r.ea, r.eb);
            }
            Out<DTO>::scalar(orow, e0 + e, d);
        }
}

// dz of one vector (element index idx*VEC..), stored; `own_y`: this vector
// holds the target, element ey, whose value the caller passes as zy.
template <int DTI, int DTO>
__device__ __forceinline__ void sweep_dz(void* orow, int64_t idx, const uint4& v, const TokenResult& r, float c3,
                                         bool neg, bool own_y, int ey, float zy) {
    constexpr int VEC = In<DTI>::VEC;
    float f[VEC];
    In<DTI>::unpack(v, f);
    float d[VEC];
    if (r.eb == 0.0f) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) d[e] = __builtin_amdgcn_exp2f(fmaf(f[e], kLog2e, -c3));
    } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) d[e] = dz_with_bonus(fmaf(f[e], kLog2e, -r.c2), r.ea, r.eb);
    }
    if (own_y) {
        const float tty = fmaf(zy, kLog2e, -r.c2);
        const float dy = r.eb == 0.0f ? fmaf(r.coef, __builtin_amdgcn_exp2f(tty), -r.coef)
                                      : dz_with_bonus(tty, r.ea, r.eb) - r.coef;
        // stored with the sign flip applied to the whole vector below
        const float dys = (r.eb == 0.0f && neg) ? -dy : dy;
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            if (e == ey) d[e] = dys;
    }
    Out<DTO>::template store<VEC>(orow, idx * VEC, d, r.eb == 0.0f && neg);
}

// A zero dlogits row for the register kernel: whole vectors with 16-byte
// non-temporal stores; with MIS the row's elements of the first and last
// (partial) vectors one at a time.
template <int DTO, int VEC, int TPR, int NK, bool MIS>
__device__ __forceinline__ void zero_row(void* orow, int tid, int ilo, unsigned nwhole, int hb, int nvec, int64_t V) {
#pragma unroll
    for (int k = 0; k < NK; ++k) {
        const int idx = k * TPR + tid;
        if ((unsigned)(idx - ilo) < nwhole) Out<DTO>::template zero<VEC>(orow, (int64_t)idx * VEC - hb);
    }
    if constexpr (MIS) {
        const int last = nvec - 1;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int idx = h == 0 ? 0 : last;
            if ((h == 0 || last > 0) && tid == idx % TPR) {
                const int e0 = idx * VEC - hb;
                for (int e = e0 < 0 ? 0 : e0; e < e0 + VEC && e < (int)V; ++e) Out<DTO>::scalar(orow, e, 0.0f);
            }
        }
    }
}

// ---------------------------------------------------------------- register-resident kernel
//
// TPR threads per token row, NV 16-byte vectors per thread in registers and
// NL more in LDS (filled by direct-to-LDS loads issued with the register
// loads, so a row that outgrows the register file is still read once).
// NG more per thread, past what registers and LDS hold, are read from memory
// in each of the two sweeps, two at a time: only that part of the row is read
// twice.
// TPR == 64: four token rows per 256-thread block, one wave each, wave-only
// reductions.  TPR > 64: one row per block, cross-wave reduction through LDS.
template <int DTI, int DTO, int TPR, int NV, bool GRAD, int NL = 0, int NG = 0, bool MIS = false>
__global__ __launch_bounds__(TPR == 64 ? 256 : TPR) void tok_reg_kernel(const TokParams p) {
    static_assert(NL == 0 || TPR == 1024, "LDS-held vectors are for the one-row-per-block path");
    static_assert(NG == 0 || (NL > 0 && NG % 2 == 0), "re-read vectors follow the LDS-held ones, in pairs");
    static_assert(!MIS || (NL == 0 && NG == 0), "rows off alignment: registers only");
    constexpr int VEC = In<DTI>::VEC;
    constexpr int WPR = TPR / 64;
    constexpr int RPB = TPR == 64 ? 4 : 1;
    const int lrow = RPB == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int tid = RPB == 1 ? (int)threadIdx.x : (int)(threadIdx.x & 63);
    const int64_t t = (int64_t)xcd_runs(blockIdx.x, gridDim.x) * RPB + lrow;
    if (t >= p.n_tok) return;   // wave-uniform (RPB > 1) or block-uniform (RPB == 1)

    const int64_t src = token_source(p, t);
    if (src < 0) {
        if (tid == 0) bad_source_outputs<GRAD>(p, t);
        return;
    }
    const char* irow = reinterpret_cast<const char*>(p.logits) + src * p.ld * In<DTI>::BYTES;
    // Row geometry.  Aligned rows: vectors 0 .. nvec-1 of the row.  MIS: the
    // 16-byte-aligned vectors covering the row, vector i holding row elements
    // i*VEC - hb .. +VEC; the first and the last hold elements outside the
    // row and are taken one element at a time; [ilo, ihi) are whole.  The
    // output row has the input row's alignment phase (the dispatch checks it).
    // An aligned vector holding one element of the row lies in the same
    // 16-byte granule, so in the same page, as that element: its other bytes
    // are read (and ignored), never written.
    // The register path only runs for nvec <= TPR * (NV + NL + NG).
    int hb = 0, nvec, ilo = 0, ihi;
    const uint4* vrow;
    if constexpr (MIS) {
        const uintptr_t ia = reinterpret_cast<uintptr_t>(irow);
        hb = (int)((ia & 15u) / In<DTI>::BYTES);
        vrow = reinterpret_cast<const uint4*>(ia - (ia & 15u));
        nvec = (int)((p.V + hb + VEC - 1) / VEC);
        ilo = 1;
        ihi = nvec - 1;
    } else {
        vrow = reinterpret_cast<const uint4*>(irow);
        nvec = (int)(p.V / VEC);
        ihi = nvec;
    }
    // whole vector idx: (unsigned)(idx - ilo) < nwhole
    const unsigned nwhole = ihi > ilo ? (unsigned)(ihi - ilo) : 0u;
    void* orow = nullptr;
    if constexpr (GRAD) {
        if (p.dlogits) orow = reinterpret_cast<char*>(p.dlogits) + src * p.ld_out * Out<DTO>::BYTES;
    }
    if (p.mask[src] == 0) {
        if (tid == 0) masked_outputs<GRAD>(p, t);
        if constexpr (GRAD) {
            if (orow) zero_row<DTO, VEC, TPR, NV + NL + NG, MIS>(orow, tid, ilo, nwhole, hb, nvec, p.V);
        }
        return;
    }

    // Target logit: read by the one lane that owns element y (it alone later
    // writes dlogits[y], so an in-place update stays ordered).
    const int32_t y = p.target[src];
    const bool ybad = (uint32_t)y >= (uint64_t)p.V;
    const int vy = ybad ? 0 : (y + hb) / VEC;
    const int own_tid = vy % TPR;
    float zy_mine = 0.0f;
    if (!ybad && tid == own_tid) zy_mine = In<DTI>::scalar(irow, y);

    // Lanes past the row end load the last vector again (in bounds); the
    // sweeps skip those elements.
    uint4 x[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) x[k] = vrow[min(k * TPR + tid, nvec - 1)];
    // Vectors NV .. NV+NL-1 of each lane go straight to LDS: one
    // global_load_lds moves the wave's 64 lanes x 16 bytes to base + 16 * lane,
    // so lane tid's vector j sits at s_tail[j * TPR + tid].
    [[maybe_unused]] __shared__ uint4 s_tail[NL > 0 ? NL * TPR : 1];
    if constexpr (NL > 0) {
        const int wave = tid >> 6;
#pragma unroll
        for (int j = 0; j < NL; ++j)
            __builtin_amdgcn_global_load_lds(vrow + min((NV + j) * TPR + tid, nvec - 1),
                                             (lds_void*)(s_tail + j * TPR + wave * 64), 16, 0, 0);
    }

    [[maybe_unused]] __shared__ float s_part[WPR][3];
    [[maybe_unused]] __shared__ float s_zy;
    float zy;
    if constexpr (WPR == 1) {
        zy = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(zy_mine), own_tid));
    } else {
        if (tid == own_tid) s_zy = zy_mine;   // read after the first barrier below
    }

    // One sweep: each lane sums 2^t and 2^t * t, t = z*log2(e) - c, with its
    // own shift c = log2(e) * (largest element of its first vector); the
    // lanes' (c, s, w) are then merged exactly.  Any shift near the lane's
    // maximum keeps the sums in range; a row where they overflow or turn NaN
    // (a -inf or NaN logit, a spread of more than ~80 nats within one lane)
    // takes the exact max-shifted sweeps instead.
    float c = -INFINITY, s = 0.0f, w = 0.0f;   // an empty lane: s = 0
    // MIS: the last (partial) vector is vector klast of lane llast
    [[maybe_unused]] const int klast = (nvec - 1) / TPR, llast = (nvec - 1) % TPR;
    if (tid < nvec) {
        float f[VEC];
        In<DTI>::unpack(x[0], f);
        float m0;
        if constexpr (MIS) {
            // lane tid's first vector is vector tid: only the row's elements
            const int elo = hb - tid * VEC, ehi = (int)p.V + hb - tid * VEC;
            m0 = -INFINITY;
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                if (e >= elo && e < ehi) m0 = fmaxf(m0, f[e]);
        } else {
            m0 = f[0];
#pragma unroll
            for (int e = 1; e < VEC; ++e) m0 = fmaxf(m0, f[e]);
        }
        c = m0 * kLog2e;
        if (!isfinite(c)) c = 0.0f;
    }
    // Each vector is fenced on its own just before its sums: a fence over the
    // whole array would make every wave wait for all of its loads before the
    // first sum, while per vector the sweep follows the loads as they land.
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int idx = k * TPR + tid;
        if ((unsigned)(idx - ilo) < nwhole) {
            opaque_vec(x[k]);
            sweep_sums<DTI>(x[k], c, s, w);
        }
        if constexpr (MIS) {
            if ((k == 0 && tid == 0) || (k == klast && tid == llast && nvec > 1)) {
                opaque_vec(x[k]);
                sweep_sums_part<DTI>(x[k], hb - idx * VEC, (int)p.V + hb - idx * VEC, c, s, w, false);
            }
        }
    }
    if constexpr (NL > 0) {
        // this wave's direct-to-LDS loads have landed (each lane reads only
        // the 16 bytes its own wave's load wrote)
        __builtin_amdgcn_s_waitcnt(GRPO_LOSS_VMCNT(0));
#pragma unroll
        for (int j = 0; j < NL; ++j)
            if ((NV + j) * TPR + tid < nvec) sweep_sums<DTI>(s_tail[j * TPR + tid], c, s, w);
    }
    // the vectors past registers and LDS (clamped loads stay in the row)
#pragma unroll
    for (int g = 0; g < NG; g += 2) {
        const int i0 = (NV + NL + g) * TPR + tid, i1 = i0 + TPR;
        const uint4 a = vrow[min(i0, nvec - 1)], b = vrow[min(i1, nvec - 1)];
        if (i0 < nvec) sweep_sums<DTI>(a, c, s, w);
        if (i1 < nvec) sweep_sums<DTI>(b, c, s, w);
    }
    block_merge<WPR>(c, s, w, tid, s_part);
    if constexpr (WPR > 1) zy = s_zy;

    if (!(isfinite(s) && isfinite(w))) {
        // exact sweeps: shift by the row maximum, clamp t so that 2^t * t of
        // a -inf logit is 0 (block-uniform branch: s and w are the same on
        // every lane)
        opaque_regs(x);
        float m = -INFINITY;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int idx = k * TPR + tid;
            if ((unsigned)(idx - ilo) < nwhole) sweep_max<DTI>(x[k], m);
            if constexpr (MIS) {
                if ((k == 0 && tid == 0) || (k == klast && tid == llast && nvec > 1))
                    sweep_max_part<DTI>(x[k], hb - idx * VEC, (int)p.V + hb - idx * VEC, m);
            }
        }
#pragma unroll
        for (int j = 0; j < NL; ++j)
            if ((NV + j) * TPR + tid < nvec) sweep_max<DTI>(s_tail[j * TPR + tid], m);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const int i = (NV + NL + g) * TPR + tid;
            if (i < nvec) sweep_max<DTI>(vrow[i], m);
        }
        m = block_max<WPR>(m, tid, s_part);
        c = m * kLog2e;
        s = 0.0f;
        w = 0.0f;
        opaque_regs(x);
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int idx = k * TPR + tid;
            if ((unsigned)(idx - ilo) < nwhole) sweep_sums_clamped<DTI>(x[k], c, s, w);
            if constexpr (MIS) {
                if ((k == 0 && tid == 0) || (k == klast && tid == llast && nvec > 1))
                    sweep_sums_part<DTI>(x[k], hb - idx * VEC, (int)p.V + hb - idx * VEC, c, s, w, true);
            }
        }
#pragma unroll
        for (int j = 0; j < NL; ++j)
            if ((NV + j) * TPR + tid < nvec) sweep_sums_clamped<DTI>(s_tail[j * TPR + tid], c, s, w);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const int i = (NV + NL + g) * TPR + tid;
            if (i < nvec) sweep_sums_clamped<DTI>(vrow[i], c, s, w);
        }
        block_sum2<WPR>(s, w, tid, s_part);
    }

    const TokenResult r = token_tail<GRAD>(p, t, src, c, s, w, zy, ybad, tid == 0);
    if constexpr (GRAD) {
        if (!orow) return;
        if (r.coef == 0.0f && r.eb == 0.0f) {   // zero advantage or clipped, no bonus: the row is zero
            zero_row<DTO, VEC, TPR, NV + NL + NG, MIS>(orow, tid, ilo, nwhole, hb, nvec, p.V);
            return;
        }
        // sweep 3: dz = coef * p, minus coef at the target.  Without the
        // bonus, coef is folded into the exponent: |coef| p_v = 2^(z_v log2(e)
        // - (c2 - log2|coef|)), and its sign goes onto the stored bits.
        opaque_regs(x);
        const float c3 = r.c2 - log2f(fabsf(r.coef));
        const bool neg = r.coef < 0.0f;
        // whole vector idx starts at row element idx*VEC - hb
        void* ovec = reinterpret_cast<char*>(orow) - (int64_t)hb * Out<DTO>::BYTES;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int idx = k * TPR + tid;
            if ((unsigned)(idx - ilo) < nwhole) sweep_dz<DTI, DTO>(ovec, idx, x[k], r, c3, neg, false, -1, 0.0f);
            if constexpr (MIS) {
                if ((k == 0 && tid == 0) || (k == klast && tid == llast && nvec > 1))
                    dz_part<DTI, DTO>(orow, (int64_t)idx * VEC - hb, x[k], r, c3, neg, hb - idx * VEC,
                                      (int)p.V + hb - idx * VEC);
            }
        }
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int idx = (NV + j) * TPR + tid;
            if (idx < nvec) sweep_dz<DTI, DTO>(orow, idx, s_tail[j * TPR + tid], r, c3, neg, false, -1, 0.0f);
        }
        // the re-read vectors: each is read and then written by the same lane,
        // so an in-place update stays ordered
#pragma unroll
        for (int g = 0; g < NG; g += 2) {
            const int i0 = (NV + NL + g) * TPR + tid, i1 = i0 + TPR;
            const uint4 a = vrow[min(i0, nvec - 1)], b = vrow[min(i1, nvec - 1)];
            if (i0 < nvec) sweep_dz<DTI, DTO>(orow, i0, a, r, c3, neg, false, -1, 0.0f);
            if (i1 < nvec) sweep_dz<DTI, DTO>(orow, i1, b, r, c3, neg, false, -1, 0.0f);
        }
        // The target element, coef * p_y - coef: rewritten by the lane that
        // owns it, after (program order) its own store of the vector holding
        // it; no vector of the sweep needs a test for the target.
        if (!ybad && tid == own_tid) {
            const float tty = fmaf(zy, kLog2e, -r.c2);
            const float dy = r.eb == 0.0f ? fmaf(r.coef, __builtin_amdgcn_exp2f(tty), -r.coef)
                                          : dz_with_bonus(tty, r.ea, r.eb) - r.coef;
            Out<DTO>::scalar(orow, y, dy);
        }
    }
}

// ---------------------------------------------------------------- paired forward kernel
//
// Forward only, with the fused loss's arithmetic: the register kernel's lane
// partition (TPR lanes per row, lane tid taking vectors k*TPR + tid in
// increasing k for k < NT = NV + NL + NG), its per-lane shift from the lane's
// first vector, its block merge and its exact fallback, so logp, lse and
// entropy come out with the fused call's bits.  The row need not stay on
// chip for a gradient sweep, so the vectors stream through a window of PB
// loads per lane (double-buffered), and two 1024-thread blocks fit a CU.
template <int DTI, int TPR, int NT, bool MIS>
__global__ __launch_bounds__(TPR == 64 ? 256 : TPR, TPR == 1024 ? 2 : 1) void tok_fwd_paired_kernel(const TokParams p) {
    constexpr int VEC = In<DTI>::VEC;
    constexpr int WPR = TPR / 64;
    constexpr int RPB = TPR == 64 ? 4 : 1;
    constexpr int PB = 4;   // loads in flight per lane (per half of the window)
    const int lrow = RPB == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int tid = RPB == 1 ? (int)threadIdx.x : (int)(threadIdx.x & 63);
    const int64_t t = (int64_t)xcd_runs(blockIdx.x, gridDim.x) * RPB + lrow;
    if (t >= p.n_tok) return;   // wave-uniform (RPB > 1) or block-uniform (RPB == 1)

    const int64_t src = token_source(p, t);
    if (src < 0) {
        if (tid == 0) bad_source_outputs<false>(p, t);
        return;
    }
    if (p.mask[src] == 0) {
        if (tid == 0) masked_outputs<false>(p, t);
        return;
    }
    const char* irow = reinterpret_cast<const char*>(p.logits) + src * p.ld * In<DTI>::BYTES;
    // row geometry as in the register kernel (aligned rows, or the aligned
    // vectors covering a row off 16-byte alignment)
    int hb = 0, nvec, ilo = 0, ihi;
    const uint4* vrow;
    if constexpr (MIS) {
        const uintptr_t ia = reinterpret_cast<uintptr_t>(irow);
        hb = (int)((ia & 15u) / In<DTI>::BYTES);
        vrow = reinterpret_cast<const uint4*>(ia - (ia & 15u));
        nvec = (int)((p.V + hb + VEC - 1) / VEC);
        ilo = 1;
        ihi = nvec - 1;
    } else {
        vrow = reinterpret_cast<const uint4*>(irow);
        nvec = (int)(p.V / VEC);
        ihi = nvec;
    }
    const unsigned nwhole = ihi > ilo ? (unsigned)(ihi - ilo) : 0u;
    [[maybe_unused]] const int klast = (nvec - 1) / TPR, llast = (nvec - 1) % TPR;

    const int32_t y = p.target[src];
    const bool ybad = (uint32_t)y >= (uint64_t)p.V;
    const int vy = ybad ? 0 : (y + hb) / VEC;
    const int own_tid = vy % TPR;
    float zy_mine = 0.0f;
    if (!ybad && tid == own_tid) zy_mine = In<DTI>::scalar(irow, y);
    [[maybe_unused]] __shared__ float s_part[WPR][3];
    [[maybe_unused]] __shared__ float s_zy;
    float zy;
    if constexpr (WPR == 1) {
        zy = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(zy_mine), own_tid));
    } else {
        if (tid == own_tid) s_zy = zy_mine;   // read after the first barrier below
    }

    // one vector of the sweep: the whole-vector sums, or the row's elements of
    // a partial vector (MIS), exactly as the register kernel takes vector k
    auto sums = [&](int k, const uint4& v, float c, float& s, float& w, bool clamped) {
        const int idx = k * TPR + tid;
        if ((unsigned)(idx - ilo) < nwhole) {
            if (clamped) sweep_sums_clamped<DTI>(v, c, s, w);
            else sweep_sums<DTI>(v, c, s, w);
        }
        if constexpr (MIS) {
            if ((k == 0 && tid == 0) || (k == klast && tid == llast && nvec > 1))
                sweep_sums_part<DTI>(v, hb - idx * VEC, (int)p.V + hb - idx * VEC, c, s, w, clamped);
        }
    };
    auto load = [&](int k) { return vrow[min(k * TPR + tid, nvec - 1)]; };

    float c = -INFINITY, s = 0.0f, w = 0.0f;
    uint4 buf[2][PB];
#pragma unroll
    for (int b = 0; b < PB; ++b)
        if (b < NT) buf[0][b] = load(b);
    if (tid < nvec) {
        float f[VEC];
        In<DTI>::unpack(buf[0][0], f);
        float m0;
        if constexpr (MIS) {
            const int elo = hb - tid * VEC, ehi = (int)p.V + hb - tid * VEC;
            m0 = -INFINITY;
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                if (e >= elo && e < ehi) m0 = fmaxf(m0, f[e]);
        } else {
            m0 = f[0];
#pragma unroll
            for (int e = 1; e < VEC; ++e) m0 = fmaxf(m0, f[e]);
        }
        c = m0 * kLog2e;
        if (!isfinite(c)) c = 0.0f;
    }
    // window i holds vectors i*PB .. i*PB+PB-1; the next window's loads are
    // issued before this window's sums
#pragma unroll
    for (int i = 0; i * PB < NT; ++i) {
        const int cur = i & 1;
        if ((i + 1) * PB < NT) {
#pragma unroll
            for (int b = 0; b < PB; ++b)
                if ((i + 1) * PB + b < NT) buf[cur ^ 1][b] = load((i + 1) * PB + b);
        }
#pragma unroll
        for (int b = 0; b < PB; ++b)
            if (i * PB + b < NT) {
                opaque_vec(buf[cur][b]);
                sums(i * PB + b, buf[cur][b], c, s, w, false);
            }
    }
    block_merge<WPR>(c, s, w, tid, s_part);
    if constexpr (WPR > 1) zy = s_zy;

    if (!(isfinite(s) && isfinite(w))) {
        // the register kernel's exact sweeps, the row read again
        float m = -INFINITY;
        for (int k = 0; k < NT; ++k) {
            const uint4 v = load(k);
            const int idx = k * TPR + tid;
            if ((unsigned)(idx - ilo) < nwhole) sweep_max<DTI>(v, m);
            if constexpr (MIS) {
                if ((k == 0 && tid == 0) || (k == klast && tid == llast && nvec > 1))
                    sweep_max_part<DTI>(v, hb - idx * VEC, (int)p.V + hb - idx * VEC, m);
            }
        }
        m = block_max<WPR>(m, tid, s_part);
        c = m * kLog2e;
        s = 0.0f;
        w = 0.0f;
        for (int k = 0; k < NT; ++k) sums(k, load(k), c, s, w, true);
        block_sum2<WPR>(s, w, tid, s_part);
    }
    token_tail<false>(p, t, src, c, s, w, zy, ybad, tid == 0);
}

// ---------------------------------------------------------------- streaming kernel
//
// Rows the register/LDS path cannot take: V beyond its capacity, or rows off
// 16-byte alignment whose dlogits rows have another dtype or another
// alignment phase.  256 threads per token
// stream the row from memory: 16-byte vectors over its aligned interior,
// single elements for the head before the first 16-byte boundary and the tail
// after the last whole vector.  The sums use the register path's per-lane
// shift and exact merge (the exact max-shifted sweeps when they overflow);
// the dz pass streams the row again, so a token costs two reads and one write
// of the row.  Interior vectors of dz are 16-byte (8-byte) stores when the
// output row shares the input row's alignment, single elements otherwise.

constexpr int kStreamTPR = 256;
constexpr int kStreamUnroll = 4;   // vectors in flight per lane (gradient path; the forward-only path keeps 8)

// Elements before the row's first 16-byte boundary (at most V), the whole
// 16-byte vectors after them, and the first element after those vectors.
struct RowGeom {
    int64_t hh;
    int64_t nvi;
    int64_t t0;
};

template <int BYTES, int VEC>
__device__ __forceinline__ RowGeom row_geom(const void* row, int64_t V) {
    const int64_t h = (int64_t)((16u - (uint32_t)(reinterpret_cast<uintptr_t>(row) & 15u)) & 15u) / BYTES;
    RowGeom g;
    g.hh = h < V ? h : V;
    g.nvi = (V - g.hh) / VEC;
    g.t0 = g.hh + g.nvi * VEC;
    return g;
}

// a zero row of V output elements, whatever the row's alignment
template <int DTO>
__device__ __forceinline__ void zero_row_stream(void* orow, int64_t V, int tid) {
    constexpr int OVEC = 16 / Out<DTO>::BYTES;   // output elements per 16-byte store
    const RowGeom g = row_geom<Out<DTO>::BYTES, OVEC>(orow, V);
    if (tid < g.hh) Out<DTO>::scalar(orow, tid, 0.0f);
    uint4* v = reinterpret_cast<uint4*>(reinterpret_cast<char*>(orow) + g.hh * Out<DTO>::BYTES);
    for (int64_t i = tid; i < g.nvi; i += kStreamTPR) st16_nt(v + i, make_uint4(0, 0, 0, 0));
    if (g.t0 + tid < V) Out<DTO>::scalar(orow, g.t0 + tid, 0.0f);
}

// 2^t and 2^t t sums of one element
__device__ __forceinline__ void elem_sums(float z, float c, float& s, float& w) {
    const float tt = fmaf(z, kLog2e, -c);
    const float ee = __builtin_amdgcn_exp2f(tt);
    s += ee;
    w = fmaf(ee, tt, w);
}

__device__ __forceinline__ void elem_sums_clamped(float z, float c, float& s, float& w) {
    const float tt = fmaf(z, kLog2e, -c);
    const float ee = __builtin_amdgcn_exp2f(tt);
    s += ee;
    w = fmaf(ee, fmaxf(tt, kNegClampLog2), w);
}

// dlogits value of element z (true value, sign applied); own_y: this is the target
__device__ __forceinline__ float elem_dz(float z, const TokenResult& r, float c3, bool neg, bool own_y) {
    const float tt = fmaf(z, kLog2e, -r.c2);
    if (own_y) {
        return r.eb == 0.0f ? fmaf(r.coef, __builtin_amdgcn_exp2f(tt), -r.coef) : dz_with_bonus(tt, r.ea, r.eb) - r.coef;
    }
    if (r.eb != 0.0f) return dz_with_bonus(tt, r.ea, r.eb);
    const float d = __builtin_amdgcn_exp2f(fmaf(z, kLog2e, -c3));
    return neg ? -d : d;
}

template <int DTI, int DTO, bool GRAD>
__global__ __launch_bounds__(kStreamTPR) void tok_stream_kernel(const TokParams p) {
    constexpr int TPR = kStreamTPR, WPR = TPR / 64, U = GRAD ? kStreamUnroll : 2 * kStreamUnroll;
    constexpr int VEC = In<DTI>::VEC;
    const int64_t t = blockIdx.x;
    if (t >= p.n_tok) return;
    const int tid = threadIdx.x;
    const int64_t src = token_source(p, t);
    if (src < 0) {
        if (tid == 0) bad_source_outputs<GRAD>(p, t);
        return;
    }
    const int64_t V = p.V;
    void* orow = nullptr;
    if constexpr (GRAD) {
        if (p.dlogits) orow = reinterpret_cast<char*>(p.dlogits) + src * p.ld_out * Out<DTO>::BYTES;
    }
    if (p.mask[src] == 0) {
        if (tid == 0) masked_outputs<GRAD>(p, t);
        if constexpr (GRAD) {
            if (orow) zero_row_stream<DTO>(orow, V, tid);
        }
        return;
    }
    const char* irow = reinterpret_cast<const char*>(p.logits) + src * p.ld * In<DTI>::BYTES;
    const RowGeom g = row_geom<In<DTI>::BYTES, VEC>(irow, V);
    const uint4* vin = reinterpret_cast<const uint4*>(irow + g.hh * In<DTI>::BYTES);
    const int32_t y = p.target[src];
    const bool ybad = (uint32_t)y >= (uint64_t)V;
    __shared__ float s_part[WPR][3];
    __shared__ float s_zy;
    if (tid == 0) s_zy = ybad ? 0.0f : In<DTI>::scalar(irow, y);   // read after the merge's barrier

    // the lane's shift: its first interior vector, else its head or tail element
    float c = -INFINITY, s = 0.0f, w = 0.0f;
    {
        float m0 = -INFINITY;
        bool any = true;
        if (tid < g.nvi) {
            sweep_max<DTI>(vin[tid], m0);
        } else if (tid < g.hh) {
            m0 = In<DTI>::scalar(irow, tid);
        } else if (g.t0 + tid < V) {
            m0 = In<DTI>::scalar(irow, g.t0 + tid);
        } else {
            any = false;
        }
        if (any) {
            c = m0 * kLog2e;
            if (!isfinite(c)) c = 0.0f;
        }
    }
    if (tid < g.hh) elem_sums(In<DTI>::scalar(irow, tid), c, s, w);
    for (int64_t i0 = tid; i0 < g.nvi; i0 += (int64_t)TPR * U) {
        // every load of the pass issued before the sums: past the row's end
        // a lane reads vector i0 again (in bounds) and skips it.  Without a
        // gradient sweep the row is read once, so the loads carry the
        // non-temporal hint (measured: 6.5-7.0 TB/s read against 5.6-5.9 with
        // the row held in registers); with one, the second read may still
        // find the row in the last-level cache.
        uint4 q[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = i0 + (int64_t)u * TPR;
            const int64_t ic = i < g.nvi ? i : i0;
            if constexpr (GRAD) q[u] = vin[ic];
            else q[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vin) + ic));
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (i0 + (int64_t)u * TPR < g.nvi) sweep_sums<DTI>(q[u], c, s, w);
    }
    if (g.t0 + tid < V) elem_sums(In<DTI>::scalar(irow, g.t0 + tid), c, s, w);
    block_merge<WPR>(c, s, w, tid, s_part);
    const float zy = s_zy;

    if (!(isfinite(s) && isfinite(w))) {
        // exact sweeps, streamed again (block-uniform branch)
        float m = -INFINITY;
        if (tid < g.hh) m = fmaxf(m, In<DTI>::scalar(irow, tid));
        for (int64_t i = tid; i < g.nvi; i += TPR) sweep_max<DTI>(vin[i], m);
        if (g.t0 + tid < V) m = fmaxf(m, In<DTI>::scalar(irow, g.t0 + tid));
        m = block_max<WPR>(m, tid, s_part);
        c = m * kLog2e;
        s = 0.0f;
        w = 0.0f;
        if (tid < g.hh) elem_sums_clamped(In<DTI>::scalar(irow, tid), c, s, w);
        for (int64_t i = tid; i < g.nvi; i += TPR) sweep_sums_clamped<DTI>(vin[i], c, s, w);
        if (g.t0 + tid < V) elem_sums_clamped(In<DTI>::scalar(irow, g.t0 + tid), c, s, w);
        block_sum2<WPR>(s, w, tid, s_part);
    }

    const TokenResult r = token_tail<GRAD>(p, t, src, c, s, w, zy, ybad, tid == 0);
    if constexpr (GRAD) {
        if (!orow) return;
        if (r.coef == 0.0f && r.eb == 0.0f) {   // zero advantage or clipped, no bonus: the row is zero
            zero_row_stream<DTO>(orow, V, tid);
            return;
        }
        const float c3 = r.c2 - log2f(fabsf(r.coef));
        const bool neg = r.coef < 0.0f;
        if (tid < g.hh) Out<DTO>::scalar(orow, tid, elem_dz(In<DTI>::scalar(irow, tid), r, c3, neg, tid == y));
        // output vectors line up with input vectors when the output row shares the input row's phase
        char* ovec = reinterpret_cast<char*>(orow) + g.hh * Out<DTO>::BYTES;
        constexpr int OALIGN = VEC * Out<DTO>::BYTES >= 16 ? 16 : 8;
        const bool oaligned = (reinterpret_cast<uintptr_t>(ovec) & (OALIGN - 1)) == 0;
        for (int64_t i0 = tid; i0 < g.nvi; i0 += (int64_t)TPR * U) {
            uint4 q[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = i0 + (int64_t)u * TPR;
                if (i < g.nvi) q[u] = vin[i];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = i0 + (int64_t)u * TPR;
                if (i >= g.nvi) continue;
                const int64_t e0 = g.hh + i * VEC;   // first element of the vector
                const bool own_y = !ybad && (int64_t)y >= e0 && (int64_t)y < e0 + VEC;
                const int ey = own_y ? (int)(y - e0) : -1;
                if (oaligned) {
                    sweep_dz<DTI, DTO>(ovec, i, q[u], r, c3, neg, own_y, ey, zy);   // elements i*VEC.. of ovec
                } else {
                    float f[VEC];
                    In<DTI>::unpack(q[u], f);
#pragma unroll
                    for (int e = 0; e < VEC; ++e) Out<DTO>::scalar(orow, e0 + e, elem_dz(f[e], r, c3, neg, e == ey));
                }
            }
        }
        if (g.t0 + tid < V)
            Out<DTO>::scalar(orow, g.t0 + tid, elem_dz(In<DTI>::scalar(irow, g.t0 + tid), r, c3, neg, g.t0 + tid == y));
    }
}

// ---------------------------------------------------------------- statistics

// One 256-thread block per row: thread j takes the row's tokens j, j+256, ...
// (eight per pass, every load of a pass issued before its adds, the adds in
// token order), then a fixed tree over the block.  A row's stats depend only
// on its own tokens (never on where the row sits in the chunk).  The row's
// objective share is s_r * (sum l - ent_coef * sum H + kl_coef * sum KL), s_r
// being the factor its tokens' gradients carried.
__global__ __launch_bounds__(256) void row_stats_kernel(const float* __restrict__ loss_tok,
                                                        const float* __restrict__ entropy,
                                                        const float* __restrict__ kl_tok,
                                                        const uint8_t* __restrict__ flags,
                                                        const int64_t* __restrict__ row_off, int64_t n_rows,
                                                        int64_t n_tok, const grpo::ObjTerms obj,
                                                        grpo_stats* __restrict__ out) {
    __shared__ double s_ls[4], s_es[4], s_ks[4];
    __shared__ long long s_nv[4], s_nc[4], s_nn[4];
    const int64_t r = blockIdx.x;
    const int i = threadIdx.x;
    if (r >= n_rows) return;
    int64_t b = row_off[r], e = row_off[r + 1];
    b = b < 0 ? 0 : (b > n_tok ? n_tok : b);
    e = e < b ? b : (e > n_tok ? n_tok : e);
    const float* kp = kl_tok ? kl_tok : loss_tok;   // read either way, added only with a KL term
    double ls = 0.0, es = 0.0, ks = 0.0;
    long long nv = 0, nc = 0, nn = 0;
    constexpr int U = 8;
    for (int64_t t0 = b + i; t0 < e; t0 += 256 * U) {
        uint8_t f[U];
        float l[U], h[U], k[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // past the row end the loads read token t0 (in bounds) and the
            // flag is cleared, so no load waits behind a branch
            const int64_t t = t0 + (int64_t)u * 256;
            const bool in = t < e;
            const int64_t tc = in ? t : t0;
            const uint8_t fl = flags[tc];
            f[u] = in ? fl : (uint8_t)0;
            l[u] = loss_tok[tc];
            h[u] = entropy[tc];
            k[u] = kp[tc];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (f[u] & 1u) {
                ls += (double)l[u];
                es += (double)h[u];
                if (kl_tok) ks += (double)k[u];
                nv += 1;
                nc += (f[u] >> 1) & 1u;
                nn += (f[u] >> 2) & 1u;
            }
        }
    }
    ls = wave_sum_d(ls);
    es = wave_sum_d(es);
    ks = wave_sum_d(ks);
    nv = wave_sum_i(nv);
    nc = wave_sum_i(nc);
    nn = wave_sum_i(nn);
    const int w = i >> 6;
    if ((i & 63) == 0) {
        s_ls[w] = ls; s_es[w] = es; s_ks[w] = ks; s_nv[w] = nv; s_nc[w] = nc; s_nn[w] = nn;
    }
    __syncthreads();
    if (i == 0) {
        grpo_stats s;
        s.loss_sum = ((s_ls[0] + s_ls[1]) + s_ls[2]) + s_ls[3];
        s.entropy_sum = ((s_es[0] + s_es[1]) + s_es[2]) + s_es[3];
        s.kl_sum = ((s_ks[0] + s_ks[1]) + s_ks[2]) + s_ks[3];
        s.n_valid = s_nv[0] + s_nv[1] + s_nv[2] + s_nv[3];
        s.n_clipped = s_nc[0] + s_nc[1] + s_nc[2] + s_nc[3];
        s.n_nonfinite = s_nn[0] + s_nn[1] + s_nn[2] + s_nn[3];
        s.n_valid_rows = s.n_valid > 0 ? 1 : 0;
        if (s.n_valid > 0) {
            const float sr = grpo_dev::token_factor(grpo_dev::step_scale(obj.scale, obj.denom), obj.row_weight,
                                                    (int32_t)r, n_rows);
            s.obj_sum = (double)sr * ((s.loss_sum - (double)obj.ent_coef * s.entropy_sum) +
                                      (double)obj.kl_coef * s.kl_sum);
        } else {
            s.obj_sum = 0.0;
        }
        out[r] = s;
    }
}

// One block: thread i sums rows i, i+256, ... in order, then a fixed tree.
__global__ __launch_bounds__(256) void chunk_stats_kernel(const grpo_stats* __restrict__ rows, int64_t n_rows,
                                                          grpo_stats* __restrict__ out) {
    __shared__ double s_ls[256], s_es[256], s_ks[256], s_os[256];
    __shared__ long long s_nv[256], s_nc[256], s_nn[256], s_nr[256];
    const int i = threadIdx.x;
    double ls = 0.0, es = 0.0, ks = 0.0, os = 0.0;
    long long nv = 0, nc = 0, nn = 0, nr = 0;
    for (int64_t r = i; r < n_rows; r += 256) {
        ls += rows[r].loss_sum;
        es += rows[r].entropy_sum;
        ks += rows[r].kl_sum;
        os += rows[r].obj_sum;
        nv += rows[r].n_valid;
        nc += rows[r].n_clipped;
        nn += rows[r].n_nonfinite;
        nr += rows[r].n_valid_rows;
    }
    s_ls[i] = ls; s_es[i] = es; s_ks[i] = ks; s_os[i] = os;
    s_nv[i] = nv; s_nc[i] = nc; s_nn[i] = nn; s_nr[i] = nr;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if (i < h) {
            s_ls[i] += s_ls[i + h]; s_es[i] += s_es[i + h];
            s_ks[i] += s_ks[i + h]; s_os[i] += s_os[i + h];
            s_nv[i] += s_nv[i + h]; s_nc[i] += s_nc[i + h];
            s_nn[i] += s_nn[i + h]; s_nr[i] += s_nr[i + h];
        }
        __syncthreads();
    }
    if (i == 0) {
        grpo_stats s;
        s.loss_sum = s_ls[0];
        s.entropy_sum = s_es[0];
        s.kl_sum = s_ks[0];
        s.obj_sum = s_os[0];
        s.n_valid = s_nv[0];
        s.n_clipped = s_nc[0];
        s.n_nonfinite = s_nn[0];
        s.n_valid_rows = s_nr[0];
        *out = s;
    }
}

// Valid tokens of rows: one wave per row (lanes stride the row's tokens).
__device__ __forceinline__ long long row_valid_count(const uint8_t* __restrict__ mask,
                                                     const int64_t* __restrict__ row_off, int64_t r, int64_t n_tok,
                                                     int lane) {
    int64_t b = row_off[r], e = row_off[r + 1];
    b = b < 0 ? 0 : (b > n_tok ? n_tok : b);
    e = e < b ? b : (e > n_tok ? n_tok : e);
    long long c = 0;
    for (int64_t t = b + lane; t < e; t += 64) c += mask[t] != 0;
    return wave_sum_i(c);
}

// B = rows holding a valid token: one 1024-thread block, wave w takes rows
// w, w+16, ..., fixed-order total.
__global__ __launch_bounds__(1024) void count_rows_kernel(const uint8_t* __restrict__ mask,
                                                          const int64_t* __restrict__ row_off, int64_t n_rows,
                                                          int64_t n_tok, int64_t* __restrict__ out) {
    __shared__ long long s_part[16];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    long long c = 0;
    for (int64_t r = wave; r < n_rows; r += 16) c += row_valid_count(mask, row_off, r, n_tok, lane) > 0 ? 1 : 0;
    if (lane == 0) s_part[wave] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        long long tot = 0;
        for (int k = 0; k < 16; ++k) tot += s_part[k];
        *out = tot;
    }
}

// Per-row aggregation weights, one wave per row.
__global__ __launch_bounds__(256) void row_weights_kernel(const uint8_t* __restrict__ mask,
                                                          const int64_t* __restrict__ row_off, int64_t n_rows,
                                                          int64_t n_tok, int mode, const int64_t* __restrict__ n_seq,
                                                          float* __restrict__ w_row) {
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (r >= n_rows) return;
    if (mode == GRPO_AGG_TOKEN_MEAN) {
        if (lane == 0) w_row[r] = 1.0f;
        return;
    }
    const long long B = *n_seq > 1 ? *n_seq : 1;
    if (mode == GRPO_AGG_SEQ_MEAN_TOKEN_SUM) {
        if (lane == 0) w_row[r] = (float)(1.0 / (double)B);
        return;
    }
    const long long L = row_valid_count(mask, row_off, r, n_tok, lane);
    if (lane == 0) w_row[r] = L > 0 ? (float)(1.0 / ((double)B * (double)L)) : 0.0f;
}

// N = number of non-zero mask bytes; one 1024-thread block, 16-byte loads
// when the mask is 16-byte aligned.
__global__ __launch_bounds__(1024) void count_valid_kernel(const uint8_t* __restrict__ mask, int64_t n,
                                                           int64_t* __restrict__ out) {
    __shared__ long long s_part[16];
    const int i = threadIdx.x;
    long long c = 0;
    int64_t done = 0;
    if ((reinterpret_cast<uintptr_t>(mask) & 15u) == 0) {
        const int64_t nv = n / 16;
        const uint4* v = reinterpret_cast<const uint4*>(mask);
        for (int64_t k = i; k < nv; k += 1024) {
            const uint4 q = v[k];
            const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t x = w4[j];
                c += ((x & 0xffu) != 0) + ((x & 0xff00u) != 0) + ((x & 0xff0000u) != 0) + ((x & 0xff000000u) != 0);
            }
        }
        done = nv * 16;
    }
    for (int64_t k = done + i; k < n; k += 1024) c += mask[k] != 0;
    c = wave_sum_i(c);
    if ((i & 63) == 0) s_part[i >> 6] = c;
    __syncthreads();
    if (i == 0) {
        long long tot = 0;
        for (int k = 0; k < 16; ++k) tot += s_part[k];
        *out = tot;
    }
}

// Determinism probe: over mask-1 tokens, count those whose two log-probs
// differ by more than `bound` (or are not finite) and take the largest
// difference.  One 1024-thread block, fixed-order totals.
__global__ __launch_bounds__(1024) void probe_compare_kernel(const float* __restrict__ a, const float* __restrict__ b,
                                                             const uint8_t* __restrict__ mask, int64_t n, float bound,
                                                             grpo_probe_stats* __restrict__ out) {
    __shared__ long long s_nv[16], s_nm[16];
    __shared__ float s_mx[16];
    const int i = threadIdx.x;
    long long nv = 0, nm = 0;
    float mx = 0.0f;
    for (int64_t t = i; t < n; t += 1024) {
        if (!mask[t]) continue;
        const float d = fabsf(a[t] - b[t]);
        nv += 1;
        nm += (d <= bound) ? 0 : 1;
        mx = fmaxf(mx, isfinite(d) ? d : INFINITY);
    }
    nv = wave_sum_i(nv);
    nm = wave_sum_i(nm);
    mx = wave_max(mx);
    if ((i & 63) == 0) {
        s_nv[i >> 6] = nv;
        s_nm[i >> 6] = nm;
        s_mx[i >> 6] = mx;
    }
    __syncthreads();
    if (i == 0) {
        grpo_probe_stats r;
        r.n_valid = 0;
        r.n_moved = 0;
        float m = 0.0f;
        for (int k = 0; k < 16; ++k) {
            r.n_valid += s_nv[k];
            r.n_moved += s_nm[k];
            m = fmaxf(m, s_mx[k]);
        }
        r.max_abs = (double)m;
        *out = r;
    }
}

// tok_src of a chunk made of batch rows laid end to end (binary search of
// the chunk's row offsets per token).
__global__ __launch_bounds__(256) void chunk_tok_src_kernel(const int64_t* __restrict__ src_row_off,
                                                            int64_t n_src_rows, const int64_t* __restrict__ rows,
                                                            int64_t n_rows, const int64_t* __restrict__ dst_row_off,
                                                            int64_t n_tok, int64_t* __restrict__ tok_src) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= n_tok) return;
    if (n_rows <= 0 || dst_row_off[0] > t) {
        tok_src[t] = -1;
        return;
    }
    int64_t lo = 0, hi = n_rows;
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        if (dst_row_off[mid] <= t) lo = mid;
        else hi = mid;
    }
    const int64_t r = rows[lo];
    tok_src[t] = (t < dst_row_off[lo + 1] && (uint64_t)r < (uint64_t)n_src_rows)
                     ? src_row_off[r] + (t - dst_row_off[lo])
                     : -1;
}

// dst[k] = src[idx[k]] for elements of EB bytes; out-of-range indices give 0.
template <typename T>
__global__ __launch_bounds__(256) void gather_kernel(const T* __restrict__ src, int64_t n_src,
                                                     const int64_t* __restrict__ idx, int64_t n, T* __restrict__ dst) {
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k >= n) return;
    const int64_t i = idx[k];
    dst[k] = (uint64_t)i < (uint64_t)n_src ? src[i] : T(0);
}

__global__ __launch_bounds__(256) void tok_row_kernel(const int64_t* __restrict__ row_off, int64_t n_rows,
                                                      int64_t n_tok, int32_t* __restrict__ tok_row) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= n_tok) return;
    // last r with row_off[r] <= t, then check t < row_off[r+1]
    int64_t lo = 0, hi = n_rows;   // answer in [0, n_rows)
    if (n_rows <= 0 || row_off[0] > t) {
        tok_row[t] = -1;
        return;
    }
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        if (row_off[mid] <= t) lo = mid;
        else hi = mid;
    }
    tok_row[t] = t < row_off[lo + 1] ? (int32_t)lo : -1;
}

// ---------------------------------------------------------------- dispatch

struct RegCfg {
    int tpr;
    int nv;
    int nl;   // 16-byte vectors per thread held in LDS
    int ng;   // 16-byte vectors per thread read in both sweeps
};

// Register-resident configurations, in order of preference; the first whose
// capacity tpr * (nv + nl + ng) covers the row's 16-byte vectors is used.
// Rows up to 6144 vectors (49 152 bf16) take 256-thread blocks with up to 24
// vectors per lane: several rows per CU, at different phases of their loads
// and sweeps, ran 10-39 % faster on all-valid rows of 24 576 .. 49 152 bf16
// than one 1024-thread block per row with 4-8 vectors per lane.
// NV stops at 19: at 1024 threads a lane has 128 VGPRs, and 19 vectors (76
// VGPRs of row data) is the most that compiles without spilling.  The last
// configuration adds 9 vectors per lane in LDS (144 KiB of the CU's 160 KiB):
// rows up to 229 376 bf16 / 114 688 fp32 logits are still read once.  The
// last one reads up to 4 more vectors per lane from memory in each sweep, so
// bf16 rows up to 262 144 logits read at most 1/8 of the row twice (gradient
// path; with fp32 logits that variant would spill, and such rows stream).
constexpr RegCfg kRegCfgs[] = {{64, 1, 0, 0},    {64, 2, 0, 0},    {64, 4, 0, 0},    {64, 8, 0, 0},
                               {256, 4, 0, 0},   {256, 8, 0, 0},   {256, 16, 0, 0},  {512, 12, 0, 0},
                               {256, 24, 0, 0},  {512, 16, 0, 0},  {1024, 8, 0, 0},  {1024, 12, 0, 0},
                               {1024, 16, 0, 0}, {1024, 19, 0, 0}, {1024, 19, 9, 0}, {1024, 19, 9, 4}};

template <int DTI, int DTO, bool GRAD>
hipError_t launch_reg(const RegCfg& c, const TokParams& p, hipStream_t st, bool mis = false) {
    const int rpb = c.tpr == 64 ? 4 : 1;
    const dim3 grid((unsigned)((p.n_tok + rpb - 1) / rpb));
    const dim3 block(c.tpr == 64 ? 256 : c.tpr);
    if constexpr (DTI == DTO) {
        if (mis) {
#define GRPO_MIS_CASE(TPR_, NV_)                                                                                 \
            if (c.tpr == TPR_ && c.nv == NV_ && c.nl == 0 && c.ng == 0) {                                        \
                hipLaunchKernelGGL((tok_reg_kernel<DTI, DTO, TPR_, NV_, GRAD, 0, 0, true>), grid, block, 0, st, p); \
                return hipGetLastError();                                                                        \
            }
            GRPO_MIS_CASE(64, 1)
            GRPO_MIS_CASE(64, 2)
            GRPO_MIS_CASE(64, 4)
            GRPO_MIS_CASE(64, 8)
            GRPO_MIS_CASE(256, 4)
            GRPO_MIS_CASE(256, 8)
            GRPO_MIS_CASE(256, 16)
            GRPO_MIS_CASE(256, 24)
            GRPO_MIS_CASE(512, 12)
            GRPO_MIS_CASE(512, 16)
            GRPO_MIS_CASE(1024, 8)
            GRPO_MIS_CASE(1024, 12)
            GRPO_MIS_CASE(1024, 16)
            GRPO_MIS_CASE(1024, 19)
#undef GRPO_MIS_CASE
            return hipErrorInvalidValue;
        }
    }
#define GRPO_REG_CASE(TPR_, NV_, NL_, NG_)                                                                  \
    if (c.tpr == TPR_ && c.nv == NV_ && c.nl == NL_ && c.ng == NG_) {                                       \
        hipLaunchKernelGGL((tok_reg_kernel<DTI, DTO, TPR_, NV_, GRAD, NL_, NG_>), grid, block, 0, st, p); \
        return hipGetLastError();                                                                           \
    }
    GRPO_REG_CASE(64, 1, 0, 0)
    GRPO_REG_CASE(64, 2, 0, 0)
    GRPO_REG_CASE(64, 4, 0, 0)
    GRPO_REG_CASE(64, 8, 0, 0)
    GRPO_REG_CASE(256, 4, 0, 0)
    GRPO_REG_CASE(256, 8, 0, 0)
    GRPO_REG_CASE(256, 16, 0, 0)
    GRPO_REG_CASE(256, 24, 0, 0)
    GRPO_REG_CASE(512, 12, 0, 0)
    GRPO_REG_CASE(512, 16, 0, 0)
    GRPO_REG_CASE(1024, 8, 0, 0)
    GRPO_REG_CASE(1024, 12, 0, 0)
    GRPO_REG_CASE(1024, 16, 0, 0)
    GRPO_REG_CASE(1024, 19, 0, 0)
    GRPO_REG_CASE(1024, 19, 9, 0)
    if constexpr (DTI == GRPO_BF16) GRPO_REG_CASE(1024, 19, 9, 4)
#undef GRPO_REG_CASE
    return hipErrorInvalidValue;
}

// The paired forward kernel for the register shape c (NT = its vectors per lane).
template <int DTI>
hipError_t launch_paired(const RegCfg& c, const TokParams& p, hipStream_t st, bool mis) {
    const int rpb = c.tpr == 64 ? 4 : 1;
    const dim3 grid((unsigned)((p.n_tok + rpb - 1) / rpb));
    const dim3 block(c.tpr == 64 ? 256 : c.tpr);
    const int nt = c.nv + c.nl + c.ng;
#define GRPO_PAIRED_CASE(TPR_, NT_)                                                                         \
    if (c.tpr == TPR_ && nt == NT_) {                                                                        \
        if (mis) hipLaunchKernelGGL((tok_fwd_paired_kernel<DTI, TPR_, NT_, true>), grid, block, 0, st, p);  \
        else hipLaunchKernelGGL((tok_fwd_paired_kernel<DTI, TPR_, NT_, false>), grid, block, 0, st, p);     \
        return hipGetLastError();                                                                            \
    }
    GRPO_PAIRED_CASE(64, 1)
    GRPO_PAIRED_CASE(64, 2)
    GRPO_PAIRED_CASE(64, 4)
    GRPO_PAIRED_CASE(64, 8)
    GRPO_PAIRED_CASE(256, 4)
    GRPO_PAIRED_CASE(256, 8)
    GRPO_PAIRED_CASE(256, 16)
    GRPO_PAIRED_CASE(256, 24)
    GRPO_PAIRED_CASE(512, 12)
    GRPO_PAIRED_CASE(512, 16)
    GRPO_PAIRED_CASE(1024, 8)
    GRPO_PAIRED_CASE(1024, 12)
    GRPO_PAIRED_CASE(1024, 16)
    GRPO_PAIRED_CASE(1024, 19)
    GRPO_PAIRED_CASE(1024, 28)
    GRPO_PAIRED_CASE(1024, 32)
#undef GRPO_PAIRED_CASE
    return hipErrorInvalidValue;
}

template <int DTI, int DTO, bool GRAD>
hipError_t launch_tok(const TokParams& p, bool vec_ok, hipStream_t st, bool mis_ok = false, bool paired = false) {
    if (p.n_tok == 0) return hipSuccess;
    // Forward only, rows past 1024 vectors stream: the row need not stay on
    // chip, and many 256-thread blocks per CU keep more reads in flight than
    // one row-resident block (V = 16 384 .. 202 048 bf16: 6.2-7.0 TB/s against
    // 4.4-5.9 for the register kernel; at 8192 the register kernel is ahead).
    // `paired` (forward only): the gradient path's choice of kernel shape, so
    // that the sums run in the same lane partition and order as the fused loss.
    const bool as_grad = GRAD || paired;
    if (vec_ok && (as_grad || p.V / In<DTI>::VEC <= 1024)) {
        const int64_t nvec = p.V / In<DTI>::VEC;
        for (const RegCfg& c : kRegCfgs) {
            if (c.ng > 0 && !(as_grad && DTI == GRPO_BF16)) continue;
            if ((int64_t)c.tpr * (c.nv + c.nl + c.ng) >= nvec) {
                if constexpr (!GRAD) {
                    if (paired) return launch_paired<DTI>(c, p, st, false);
                }
                return launch_reg<DTI, DTO, GRAD>(c, p, st);
            }
        }
    }
    // Rows off 16-byte alignment whose gradient rows share their alignment
    // phase (in place, or the same dtype, stride and base phase): the register
    // kernel over the aligned vectors that cover each row, the row still read
    // once.  A row spans at most V / VEC + 1 such vectors.
    if (as_grad && DTI == DTO && !vec_ok && mis_ok) {
        const int64_t nvec = (p.V + 2 * In<DTI>::VEC - 2) / In<DTI>::VEC;
        for (const RegCfg& c : kRegCfgs) {
            if (c.nl > 0 || c.ng > 0) continue;
            if ((int64_t)c.tpr * c.nv >= nvec) {
                if constexpr (!GRAD) {
                    if (paired) return launch_paired<DTI>(c, p, st, true);
                }
                return launch_reg<DTI, DTO, GRAD>(c, p, st, true);
            }
        }
    }
    hipLaunchKernelGGL((tok_stream_kernel<DTI, DTO, GRAD>), dim3((unsigned)p.n_tok), dim3(kStreamTPR), 0, st, p);
    return hipGetLastError();
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

int check_launch(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(GRPO_EDEVICE, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

// Row stats then chunk stats for a chunk whose per-token outputs are written.
int grpo::launch_stats(void* stream, const float* loss_tok, const float* entropy, const float* kl_tok,
                       const uint8_t* flags, const int64_t* row_off, int64_t n_rows, int64_t n_tok,
                       const ObjTerms& obj, grpo_stats* row_stats, grpo_stats* chunk_stats) {
    hipStream_t st = (hipStream_t)stream;
    if (n_rows > 0) {
        hipLaunchKernelGGL(row_stats_kernel, dim3((unsigned)n_rows), dim3(256), 0, st, loss_tok, entropy, kl_tok,
                           flags, row_off, n_rows, n_tok, obj, row_stats);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return check_launch(e, "row stats");
    }
    hipLaunchKernelGGL(chunk_stats_kernel, dim3(1), dim3(256), 0, st, row_stats, n_rows, chunk_stats);
    return check_launch(hipGetLastError(), "chunk stats");
}

// ---------------------------------------------------------------- C ABI

extern "C" int grpo_count_valid(void* stream, const uint8_t* mask, int64_t n_tok, int64_t* n_valid) {
    if (n_tok < 0 || !n_valid || (n_tok > 0 && !mask)) return fail(GRPO_EINVAL, "grpo_count_valid: bad arguments");
    hipLaunchKernelGGL(count_valid_kernel, dim3(1), dim3(1024), 0, (hipStream_t)stream, mask, n_tok, n_valid);
    return check_launch(hipGetLastError(), "grpo_count_valid");
}

extern "C" int grpo_count_rows(void* stream, const uint8_t* mask, const int64_t* row_off, int64_t n_rows,
                               int64_t n_tok, int64_t* n_seq) {
    if (n_rows < 0 || n_tok < 0 || !n_seq || !row_off || (n_tok > 0 && !mask))
        return fail(GRPO_EINVAL, "grpo_count_rows: bad arguments");
    hipLaunchKernelGGL(count_rows_kernel, dim3(1), dim3(1024), 0, (hipStream_t)stream, mask, row_off, n_rows, n_tok,
                       n_seq);
    return check_launch(hipGetLastError(), "grpo_count_rows");
}

extern "C" int grpo_row_weights(void* stream, const uint8_t* mask, const int64_t* row_off, int64_t n_rows,
                                int64_t n_tok, int32_t mode, const int64_t* n_seq, float* w_row) {
    if (mode != GRPO_AGG_TOKEN_MEAN && mode != GRPO_AGG_SEQ_MEAN_TOKEN_SUM && mode != GRPO_AGG_SEQ_MEAN_TOKEN_MEAN)
        return fail(GRPO_EINVAL, "grpo_row_weights: unknown aggregation mode %d", mode);
    if (n_rows < 0 || n_tok < 0 || (n_rows > 0 && (!row_off || !w_row || !n_seq)) || (n_tok > 0 && !mask))
        return fail(GRPO_EINVAL, "grpo_row_weights: bad arguments");
    if (n_rows > 0x7fffffffLL * 4) return fail(GRPO_EINVAL, "grpo_row_weights: too many rows for one launch");
    if (n_rows == 0) return ok();
    hipLaunchKernelGGL(row_weights_kernel, dim3((unsigned)((n_rows + 3) / 4)), dim3(256), 0, (hipStream_t)stream,
                       mask, row_off, n_rows, n_tok, (int)mode, n_seq, w_row);
    return check_launch(hipGetLastError(), "grpo_row_weights");
}

extern "C" int grpo_probe_compare(void* stream, const float* recorded, const float* rescored, const uint8_t* mask,
                                  int64_t n_tok, float bound, grpo_probe_stats* out) {
    if (n_tok < 0 || !out || (n_tok > 0 && (!recorded || !rescored || !mask)) || !(bound >= 0.0f))
        return fail(GRPO_EINVAL, "grpo_probe_compare: bad arguments");
    hipLaunchKernelGGL(probe_compare_kernel, dim3(1), dim3(1024), 0, (hipStream_t)stream, recorded, rescored, mask,
                       n_tok, bound, out);
    return check_launch(hipGetLastError(), "grpo_probe_compare");
}

extern "C" int grpo_chunk_tok_src(void* stream, const int64_t* src_row_off, int64_t n_src_rows, const int64_t* rows,
                                  int64_t n_rows, const int64_t* dst_row_off, int64_t n_tok, int64_t* tok_src) {
    if (n_tok < 0 || n_rows < 0 || n_src_rows < 0 ||
        (n_tok > 0 && (!tok_src || !dst_row_off || (n_rows > 0 && (!rows || !src_row_off)))))
        return fail(GRPO_EINVAL, "grpo_chunk_tok_src: bad arguments");
    if (n_tok == 0) return ok();
    if ((n_tok + 255) / 256 > 0x7fffffffLL) return fail(GRPO_EINVAL, "grpo_chunk_tok_src: too many tokens");
    hipLaunchKernelGGL(chunk_tok_src_kernel, dim3((unsigned)((n_tok + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, src_row_off, n_src_rows, rows, n_rows, dst_row_off, n_tok, tok_src);
    return check_launch(hipGetLastError(), "grpo_chunk_tok_src");
}

extern "C" int grpo_gather(void* stream, const void* src, int64_t n_src, const int64_t* idx, int64_t n,
                           int64_t elem_bytes, void* dst) {
    if (n < 0 || n_src < 0 || (n > 0 && (!idx || !dst || (n_src > 0 && !src))))
        return fail(GRPO_EINVAL, "grpo_gather: bad arguments");
    if (n == 0) return ok();
    if ((n + 255) / 256 > 0x7fffffffLL) return fail(GRPO_EINVAL, "grpo_gather: too many elements");
    const dim3 g((unsigned)((n + 255) / 256)), b(256);
    hipStream_t st = (hipStream_t)stream;
    switch (elem_bytes) {
        case 1: hipLaunchKernelGGL(gather_kernel<uint8_t>, g, b, 0, st, (const uint8_t*)src, n_src, idx, n, (uint8_t*)dst); break;
        case 2: hipLaunchKernelGGL(gather_kernel<uint16_t>, g, b, 0, st, (const uint16_t*)src, n_src, idx, n, (uint16_t*)dst); break;
        case 4: hipLaunchKernelGGL(gather_kernel<uint32_t>, g, b, 0, st, (const uint32_t*)src, n_src, idx, n, (uint32_t*)dst); break;
        case 8: hipLaunchKernelGGL(gather_kernel<uint64_t>, g, b, 0, st, (const uint64_t*)src, n_src, idx, n, (uint64_t*)dst); break;
        default: return fail(GRPO_EINVAL, "grpo_gather: elem_bytes must be 1, 2, 4 or 8");
    }
    return check_launch(hipGetLastError(), "grpo_gather");
}

extern "C" int grpo_tok_row(void* stream, const int64_t* row_off, int64_t n_rows, int64_t n_tok, int32_t* tok_row) {
    if (n_tok < 0 || n_rows < 0 || (n_tok > 0 && (!tok_row || !row_off)))
        return fail(GRPO_EINVAL, "grpo_tok_row: bad arguments");
    if (n_tok == 0) return ok();
    hipLaunchKernelGGL(tok_row_kernel, dim3((unsigned)((n_tok + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                       row_off, n_rows, n_tok, tok_row);
    return check_launch(hipGetLastError(), "grpo_tok_row");
}

namespace {

int logprob_fwd(const char* who, bool paired, void* stream, int32_t dtype, const void* logits, int64_t ld,
                int64_t n_tok, int64_t V, const int32_t* target, const uint8_t* mask, float* logp, float* lse,
                float* entropy) {
    if (dtype != GRPO_F32 && dtype != GRPO_BF16) return fail(GRPO_EINVAL, "%s: unknown dtype %d", who, dtype);
    if (n_tok < 0 || V < 1 || ld < V) return fail(GRPO_EINVAL, "%s: need n_tok >= 0, V >= 1, ld >= V", who);
    if (n_tok > 0 && (!logits || !target || !mask || !logp)) return fail(GRPO_EINVAL, "%s: NULL pointer", who);
    if (n_tok > 0x7fffffffLL) return fail(GRPO_EINVAL, "%s: too many tokens for one launch", who);
    TokParams p{};
    p.logits = logits; p.ld = ld; p.n_tok = n_tok; p.V = V;
    p.target = target; p.mask = mask;
    p.logp = logp; p.lse = lse; p.entropy = entropy;
    const int vec = dtype == GRPO_BF16 ? 8 : 4;
    const int in_b = dtype == GRPO_BF16 ? 2 : 4;
    const bool vec_ok = aligned16(logits) && ld % vec == 0 && V % vec == 0;
    // rows off alignment: the fused loss keeps them in registers when its
    // dlogits rows share their phase (in place), which the paired pass assumes
    const bool mis_ok = paired && (reinterpret_cast<uintptr_t>(logits) % in_b) == 0;
    hipError_t e = dtype == GRPO_BF16
                       ? launch_tok<GRPO_BF16, GRPO_BF16, false>(p, vec_ok, (hipStream_t)stream, mis_ok, paired)
                       : launch_tok<GRPO_F32, GRPO_F32, false>(p, vec_ok, (hipStream_t)stream, mis_ok, paired);
    return check_launch(e, who);
}

}  // namespace

extern "C" int grpo_logprob_fwd(void* stream, int32_t dtype, const void* logits, int64_t ld, int64_t n_tok,
                                int64_t V, const int32_t* target, const uint8_t* mask, float* logp, float* lse,
                                float* entropy) {
    return logprob_fwd("grpo_logprob_fwd", false, stream, dtype, logits, ld, n_tok, V, target, mask, logp, lse,
                       entropy);
}

extern "C" int grpo_logprob_fwd_paired(void* stream, int32_t dtype, const void* logits, int64_t ld, int64_t n_tok,
                                       int64_t V, const int32_t* target, const uint8_t* mask, float* logp,
                                       float* lse, float* entropy) {
    return logprob_fwd("grpo_logprob_fwd_paired", true, stream, dtype, logits, ld, n_tok, V, target, mask, logp,
                       lse, entropy);
}

extern "C" int grpo_loss_fwd_bwd(void* stream, const grpo_loss_args* a) {
    if (!a) return fail(GRPO_EINVAL, "grpo_loss_fwd_bwd: NULL args");
    if (a->struct_size != (int32_t)sizeof(grpo_loss_args))
        return fail(GRPO_EINVAL, "grpo_loss_fwd_bwd: struct_size %d != %d", a->struct_size, (int)sizeof(grpo_loss_args));
    const int di = a->in_dtype, dout = a->out_dtype;
    if ((di != GRPO_F32 && di != GRPO_BF16) || (dout != GRPO_F32 && dout != GRPO_BF16))
        return fail(GRPO_EINVAL, "grpo_loss_fwd_bwd: unknown dtype");
    if (a->n_tok < 0 || a->V < 1 || a->ld < a->V || a->n_rows < 0)
        return fail(GRPO_EINVAL, "grpo_loss_fwd_bwd: need n_tok >= 0, V >= 1, ld >= V, n_rows >= 0");
    if (a->n_tok > 0 && a->n_rows < 1) return fail(GRPO_EINVAL, "grpo_loss_fwd_bwd: tokens without rows");
    if (a->n_tok > 0x7fffffffLL || a->n_rows > 0x7fffffffLL)
        return fail(GRPO_EINVAL, "grpo_loss_fwd_bwd: too many tokens or rows for one launch");
    if (a->flags & ~GRPO_LOSS_DEFER_STATS) return fail(GRPO_EINVAL, "grpo_loss_fwd_bwd: unknown flags %d", a->flags);
    const bool defer = (a->flags & GRPO_LOSS_DEFER_STATS) != 0;
    if (!defer && (!a->chunk_stats || (a->n_rows > 0 && (!a->row_stats || !a->row_off))))
        return fail(GRPO_EINVAL, "grpo_loss_fwd_bwd: NULL stats pointer");
    if (a->n_tok > 0 && (!a->logits || !a->target || !a->mask || !a->old_logp || !a->tok_row || !a->adv_row ||
                         !a->logp || !a->entropy || !a->loss_tok || !a->tok_flags))
        return fail(GRPO_EINVAL, "grpo_loss_fwd_bwd: NULL pointer");
    if (!(a->eps_low >= 0.0f && a->eps_low <= 1.0f && a->eps_high >= 0.0f && std::isfinite(a->eps_high)))
        return fail(GRPO_EINVAL, "grpo_loss_fwd_bwd: need 0 <= eps_low <= 1 and finite eps_high >= 0");
    if (!std::isfinite(a->scale)) return fail(GRPO_EINVAL, "grpo_loss_fwd_bwd: scale must be finite");
    {
        const int rc = grpo::check_terms("grpo_loss_fwd_bwd", a->n_tok, a->ref_logp, a->kl_tok, a->ent_coef,
                                         a->kl_coef, a->kl_type);
        if (rc != GRPO_OK) return rc;
    }
    const int in_b = di == GRPO_BF16 ? 2 : 4, out_b = dout == GRPO_BF16 ? 2 : 4;
    if (a->tok_src && a->n_src < 1) return fail(GRPO_EINVAL, "grpo_loss_fwd_bwd: tok_src needs n_src >= 1");
    if (a->dlogits && a->n_tok > 0) {
        if (a->ld_out < a->V) return fail(GRPO_EINVAL, "grpo_loss_fwd_bwd: ld_out < V");
        // rows that may be touched: the chunk's own, or every batch row behind tok_src
        const int64_t span = a->tok_src ? a->n_src : a->n_tok;
        const uintptr_t i0 = (uintptr_t)a->logits, i1 = i0 + (uintptr_t)((span - 1) * a->ld + a->V) * in_b;
        const uintptr_t o0 = (uintptr_t)a->dlogits, o1 = o0 + (uintptr_t)((span - 1) * a->ld_out + a->V) * out_b;
        const bool overlap = o0 < i1 && i0 < o1;
        if (overlap && !(o0 == i0 && di == dout && a->ld == a->ld_out))
            return fail(GRPO_EINVAL, "grpo_loss_fwd_bwd: dlogits overlaps logits without being the same buffer");
    }
    TokParams p{};
    p.logits = a->logits; p.ld = a->ld; p.n_tok = a->n_tok; p.V = a->V;
    p.target = a->target; p.mask = a->mask; p.old_logp = a->old_logp;
    p.tok_row = a->tok_row; p.adv_row = a->adv_row; p.n_rows = a->n_rows;
    p.eps_low = a->eps_low; p.eps_high = a->eps_high; p.scale = a->scale; p.denom = a->denom;
    p.dlogits = a->dlogits; p.ld_out = a->ld_out;
    p.logp = a->logp; p.lse = a->lse; p.entropy = a->entropy; p.loss_tok = a->loss_tok; p.tok_flags = a->tok_flags;
    p.terms = grpo_dev::Terms{a->row_weight, a->ref_logp, a->ent_coef, a->kl_coef, a->kl_type};
    p.kl_tok = a->ref_logp ? a->kl_tok : nullptr;
    p.tok_src = a->tok_src;
    p.n_src = a->n_src;
    const int vec = di == GRPO_BF16 ? 8 : 4;
    bool vec_ok = aligned16(a->logits) && a->ld % vec == 0 && a->V % vec == 0;
    if (a->dlogits) vec_ok = vec_ok && aligned16(a->dlogits) && (a->ld_out * out_b) % 16 == 0 && ((int64_t)vec * out_b) % 8 == 0;
    // rows off alignment, each gradient row in its logits row's alignment phase
    // (every row: same base phase and the same stride in bytes modulo 16)
    const bool mis_ok = di == dout && (reinterpret_cast<uintptr_t>(a->logits) % in_b) == 0 &&
                        (!a->dlogits || ((reinterpret_cast<uintptr_t>(a->dlogits) - reinterpret_cast<uintptr_t>(a->logits)) % 16 == 0 &&
                                         ((a->ld_out - a->ld) * in_b) % 16 == 0));
    hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    if (di == GRPO_BF16 && dout == GRPO_BF16) e = launch_tok<GRPO_BF16, GRPO_BF16, true>(p, vec_ok, st, mis_ok);
    else if (di == GRPO_BF16) e = launch_tok<GRPO_BF16, GRPO_F32, true>(p, vec_ok, st);
    else if (dout == GRPO_BF16) e = launch_tok<GRPO_F32, GRPO_BF16, true>(p, vec_ok, st);
    else e = launch_tok<GRPO_F32, GRPO_F32, true>(p, vec_ok, st, mis_ok);
    if (e != hipSuccess) return check_launch(e, "grpo_loss_fwd_bwd (token kernel)");
    if (defer) return ok();
    const grpo::ObjTerms obj{a->scale, a->denom, a->row_weight, a->ent_coef, a->ref_logp ? a->kl_coef : 0.0f};
    return grpo::launch_stats(stream, a->loss_tok, a->entropy, p.kl_tok, a->tok_flags, a->row_off, a->n_rows,
                              a->n_tok, obj, a->row_stats, a->chunk_stats);
}

extern "C" int grpo_loss_stats(void* stream, const grpo_loss_args* a) {
    if (!a) return fail(GRPO_EINVAL, "grpo_loss_stats: NULL args");
    if (a->struct_size != (int32_t)sizeof(grpo_loss_args))
        return fail(GRPO_EINVAL, "grpo_loss_stats: struct_size %d != %d", a->struct_size, (int)sizeof(grpo_loss_args));
    if (a->n_tok < 0 || a->n_rows < 0 || (a->n_tok > 0 && a->n_rows < 1))
        return fail(GRPO_EINVAL, "grpo_loss_stats: need n_tok >= 0 and rows for the tokens");
    if (a->n_tok > 0x7fffffffLL || a->n_rows > 0x7fffffffLL)
        return fail(GRPO_EINVAL, "grpo_loss_stats: too many tokens or rows for one launch");
    if (!a->chunk_stats || (a->n_rows > 0 && (!a->row_stats || !a->row_off)))
        return fail(GRPO_EINVAL, "grpo_loss_stats: NULL stats pointer");
    if (a->n_tok > 0 && (!a->entropy || !a->loss_tok || !a->tok_flags || (a->ref_logp && !a->kl_tok)))
        return fail(GRPO_EINVAL, "grpo_loss_stats: NULL per-token output");
    if (!std::isfinite(a->scale) || !std::isfinite(a->ent_coef) || !std::isfinite(a->kl_coef))
        return fail(GRPO_EINVAL, "grpo_loss_stats: scale, ent_coef and kl_coef must be finite");
    const grpo::ObjTerms obj{a->scale, a->denom, a->row_weight, a->ent_coef, a->ref_logp ? a->kl_coef : 0.0f};
    return grpo::launch_stats(stream, a->loss_tok, a->entropy, a->ref_logp ? a->kl_tok : nullptr, a->tok_flags,
                              a->row_off, a->n_rows, a->n_tok, obj, a->row_stats, a->chunk_stats);
}

// Shared argument checks of the extra terms.
int grpo::check_terms(const char* who, int64_t n_tok, const float* ref_logp, const float* kl_tok, float ent_coef,
                      float kl_coef, int32_t kl_type) {
    if (!std::isfinite(ent_coef) || !std::isfinite(kl_coef))
        return fail(GRPO_EINVAL, "%s: ent_coef and kl_coef must be finite", who);
    if (kl_coef != 0.0f && !ref_logp) return fail(GRPO_EINVAL, "%s: kl_coef needs ref_logp", who);
    if (ref_logp && kl_type != GRPO_KL_K1 && kl_type != GRPO_KL_K2 && kl_type != GRPO_KL_K3)
        return fail(GRPO_EINVAL, "%s: unknown kl_type %d", who, kl_type);
    if (ref_logp && n_tok > 0 && !kl_tok) return fail(GRPO_EINVAL, "%s: ref_logp needs a kl_tok output", who);
    return ok();
}
