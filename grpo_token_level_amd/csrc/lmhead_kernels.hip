// LM-head variant of the token-level GRPO loss for gfx950: the logits
// z = h W^T are produced by bf16 MFMA GEMMs tile by tile and consumed in the
// GEMM epilogues, so no [tokens x V] logit or gradient matrix is ever held.
//
// Sources: [P1] "Sizing mini-batches and micro-batches" ("The problem": the
// materialised log-softmax is the memory wall; "The hard part: deferred
// normalization": chunk gradients add up to the step gradient); [P4] "How a
// context-compaction step fits a variable number of rows into one batch"
// (rows are micro-batched, padding rows are masked and add nothing).
//
// One call handles one micro-batch chunk of n tokens.  Masked tokens (pads,
// observations) contribute nothing, so a one-block kernel first lists the
// chunk's valid tokens on the device (index map + count); every GEMM below
// runs over those rows only.  Grids are sized for all n tokens and tiles past
// the device count exit at once, so the host never waits for the count.
//   pass 1  GEMM z = h W^T over the whole vocabulary; the epilogue reduces
//           each 64-column slice of a token row to (max, sum e, sum e*t) and
//           picks out the target logit.  A merge kernel combines the slices
//           (fixed order) into logsumexp, entropy, log-prob, the surrogate and
//           the gradient coefficient.
//           With a caller workspace the epilogue also stores z (fp32) of
//           the valid tokens.
//   pass 2  per vocabulary chunk: dz = coef*(softmax - onehot) in bf16
//           (row-major and transposed) into the workspace, from the stored z
//           by an elementwise kernel, or (the fixed-scratch entry point, in
//           chunks of at most 65536 columns) by a GEMM that recomputes z and
//           forms dz in its epilogue; both take the same arithmetic on the
//           same fp32 z, so dz has the same bits either way.  Then dh (+)=
//           dz W_c (split-K, one fp32 partial per split, summed in order at
//           the end) and dW_c += dz^T h, two more MFMA GEMMs with fp32
//           accumulation.
// All products use one kernel shape, C[m,n] = sum_k A[m,k] B[n,k] with both
// operands K-contiguous ("NT"): W for pass 1, W^T for dh, h^T and dz^T for dW.
//
// MFMA: v_mfma_f32_32x32x16_bf16.  A 512-thread block computes a 256x256 tile
// (eight waves in 4 x 2, each 64x128 = 2x4 MFMA tiles).  K advances 64 at a
// time through two LDS stages of 64 KiB (one loading while the other feeds
// the MFMAs), filled by global_load_lds (16 bytes per lane straight into
// LDS, no register staging; a tile row is one 128-byte line per stage); rows
// past the edge and k past the end load from a zero page.  Lane layouts (checked on the device): operand lane
// l holds row/column l%32 and k = (l/32)*8 .. +8; result lane l, register i
// holds column l%32 and row (i/4)*8 + (l/32)*4 + i%4.  Blocks are mapped so
// that each XCD works through a contiguous range of tiles, the index with
// fewer tiles fastest: the tiles that share a slice of the larger operand (W in
// pass 1, dz^T for dW) run together on one L2.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "common.h"
#include "surrogate.h"

using grpo::fail;
using grpo::ok;
using grpo_dev::kLn2;
using grpo_dev::kLog2e;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 256, BN = 256;    // block tile
constexpr int BK = 64;               // k per LDS stage (one 128-byte line per tile row)
constexpr int NST = 2;               // LDS stages: one loading while the other is consumed
constexpr int NTHREADS = 512;        // eight waves in 4 (M) x 2 (N), each owning a 64 x 128 sub-tile
constexpr int WM = 64, WN = 128;     // wave tile
constexpr int FM = WM / 32, FN = WN / 32;
constexpr int ROWB = BK * 2;         // bytes of one tile row in one stage
constexpr int OPB = BM * ROWB;       // bytes of one operand in one stage (32 KiB)
constexpr int STB = 2 * OPB;         // bytes of one stage (64 KiB)
constexpr int EPI_ROW_Q = WN + 4;    // floats per row of a wave's epilogue buffer (16-byte reads)
constexpr int EPIB = 8 * 32 * EPI_ROW_Q * 4;
constexpr int SMEM = NST * STB > EPIB ? NST * STB : EPIB;
constexpr int DZT_ROWB = 64 * 2 + 8;  // bytes per column of a wave's dz^T staging (64 tokens + 8: conflict-free writes)
constexpr int DZT_OFF = 8192;         // the staging follows the per-token factors
constexpr int DZR_ROWB = WN * 2 + 16; // bytes per token row of a wave's dz staging (128 columns + 16)
constexpr int DZ_WAVEB = 64 * DZR_ROWB > WN * DZT_ROWB ? 64 * DZR_ROWB : WN * DZT_ROWB;   // one buffer, used twice
constexpr int SMEM_DZ = DZT_OFF + 8 * DZ_WAVEB > SMEM ? DZT_OFF + 8 * DZ_WAVEB : SMEM;
constexpr int NXCD = 8;
constexpr int kVocabChunkMax = 65536;   // pass-2 vocabulary chunk bound (sizes the dz workspace)
constexpr int kVocabChunkMin = 16384;
constexpr int kDhSplitMax = 16;         // dh split-K partials (sizes the dh workspace)
constexpr int kTokPad = 64;             // token count padding of h^T and dz^T rows (128-byte rows)
constexpr int64_t kMaxTokens = 65535LL * 64;   // tokens per call (the h^T transpose grid's y extent)

typedef __attribute__((address_space(3))) void lds_void;

// Source of the direct-to-LDS loads for rows beyond M / N and k beyond the
// split: sixteen zero bytes (the loader zero-fills device globals).
__device__ __attribute__((aligned(64))) uint16_t g_zero_page[32];

enum { EPI_STATS = 0, EPI_DZ = 1, EPI_ACC = 2 };

// Measured rates behind the pass-2 cost model: a 256 x 256 x 64 block step
// takes ~2 us at ~1 PFLOP/s; HBM moves ~5 bytes per ns.
constexpr float kKstepUs = 2.0f, kHbmBytesPerUs = 5.0e6f;

// The dh GEMM's split-K count, chosen on the device from the chunk's valid
// rows (the host plan counts every token, pads included, and a mostly padded
// chunk would leave most compute units idle): the count s <= cap minimising
// rounds(tiles(rows) * s blocks on cus compute units) x the k-steps of the
// widest vocabulary chunk split s ways, over the call's chunks, plus the HBM
// time of the s fp32 partials.  The same for every chunk of a call, and
// recomputed identically by the sum of the partials.
struct SplitRule {
    int cap;       // 0: off (GemmArgs ksplit / kper hold)
    int kref;      // width of the widest vocabulary chunk
    int chunks;    // vocabulary chunks in the call
    int cus;       // compute units
    int tiles_n;   // tiles along H
    int cols;      // H
};

__device__ __forceinline__ int dev_split_count(const SplitRule& r, int rows) {
    const int tiles = (rows + BM - 1) / BM * r.tiles_n;
    int best = 1;
    float best_cost = -1.0f;
    for (int sp = 1; sp <= r.cap; ++sp) {
        const float rounds = (float)((tiles * sp + r.cus - 1) / r.cus);
        const float ks = (float)(((r.kref + sp - 1) / sp + BK - 1) / BK);
        const float partials = 2.0f * (float)r.chunks * (float)sp * (float)rows * (float)r.cols * 4.0f;
        const float cost = rounds * ks * (float)r.chunks + partials / (kHbmBytesPerUs * kKstepUs);
        // a split must save at least 1 % to be worth its partial
        if (best_cost < 0.0f || cost * 100.0f < best_cost * 99.0f) {
            best_cost = cost;
            best = sp;
        }
    }
    return best;
}

struct GemmArgs {
    const uint16_t* A;   // row m at A + m*lda (A + a_rows[m]*lda with a row map), K contiguous
    int64_t lda;
    const uint16_t* B;   // row n at B + n*ldb, K contiguous
    int64_t ldb;
    int M, N, K;         // K % 8 == 0; rows >= M / >= N are read as zeros
    // Valid-token compaction (NULL = off).  The grid is sized for the host
    // bounds M / K; the device count *m_dev (rows, <= M) or the device count
    // *k_dev rounded up to kTokPad (K, <= K) takes their place in the kernel,
    // and tiles past it exit at once.
    const int32_t* a_rows;   // A row (and target index) of row m
    const int32_t* m_dev;
    const int32_t* k_dev;
    int tiles_m, tiles_n;
    int ksplit, kper;    // K range of split s: [s*kper, min(K, (s+1)*kper)), kper % BK == 0
    int n_fast;          // tile order: N index fastest (else M fastest)
    SplitRule split;     // cap > 0: tiles from the device row count, split count by the rule (ksplit sizes
                         // the grid: at least the rule's cap)
    // EPI_STATS
    float4* part;        // part[m * n_parts + n/64] = {max, sum e, sum e*t, 0}
    int n_parts;
    const int32_t* target;
    float* zy;           // zy[m] = z[m, target[m]]
    float* zst;          // NULL, or z itself: zst[m * ld_zst + n] (fp32, for pass 2 without a recompute)
    int64_t ld_zst;
    // EPI_DZ (per-token arrays indexed by row m; target by the A row)
    const float* c2;     // log2-domain logsumexp per token
    const float* coef;   // gradient coefficient per token
    const float* ea;     // with the entropy bonus (bonus != 0): dz = p * (ea + eb * t) - coef * onehot,
    const float* eb;     //   t = z*log2e - c2, per token
    int bonus;
    int col0;            // vocabulary index of column 0 of this chunk
    int m_out;           // rows [M, m_out) are written as zeros (K padding of dz^T);
                         // with m_dev, m_out = *m_dev rounded up to kTokPad
    uint16_t* dz;        // dz[m * ld_dz + n]
    int64_t ld_dz;
    uint16_t* dzT;       // dzT[n * ld_dzT + koff + m]
    int64_t ld_dzT;
    const int32_t* dzT_off;   // NULL (koff = 0), or the device column offset koff (a dW window's fill)
    // EPI_ACC
    float* C;            // split s: (C + s*c_split)[m * ldc + n] = (beta ? that : 0) + acc
    int64_t ldc;
    int64_t c_split;
    int beta;
    const uint16_t* zero;   // device address of g_zero_page (set by launch_gemm)
};

__device__ __forceinline__ uint16_t to_bf16(float x) {
    f32x2 v = {x, 0.0f};
    bf16x2 r = __builtin_convertvector(v, bf16x2);
    return (uint16_t)(__builtin_bit_cast(uint32_t, r) & 0xffffu);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Hardware dispatch sends block b to XCD b % 8; renumber so that XCD x owns a
// contiguous range of logical tiles (a bijection for any block count).
__device__ __forceinline__ int xcd_logical(int b, int nb) {
    const int q = nb / NXCD, r = nb % NXCD;
    const int x = b % NXCD, i = b / NXCD;
    return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// LDS rows are 128 bytes (eight 16-byte k chunks); chunk c of row r is
// stored at position c ^ swz(r).  A 16-byte LDS read serves 16 lanes per
// pass over 64 banks (256 bytes), i.e. two 128-byte rows: the eight rows of
// one parity among 16 consecutive rows must take eight different positions,
// and so must any eight consecutive rows (measured: the plain r & 7 pattern
// left two-way conflicts on every fragment read).
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their no-wait maxima)
#define GRPO_VMCNT(n) (((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

template <int EPI>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_nt_kernel(const GemmArgs g) {
    __shared__ __attribute__((aligned(1024))) char smem[EPI == EPI_DZ ? SMEM_DZ : SMEM];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int M = g.m_dev ? min(g.M, *g.m_dev) : g.M;
    int tiles_m = g.tiles_m, ksplit = g.ksplit, kper = g.kper, n_fast = g.n_fast;
    if (g.split.cap > 0) {
        // only the valid rows' tiles, split by the rule; the active blocks are
        // the grid's first, spread over the XCDs like a grid of their own
        tiles_m = (M + BM - 1) / BM;
        ksplit = dev_split_count(g.split, M);
        kper = ((g.K + ksplit - 1) / ksplit + BK - 1) / BK * BK;
        n_fast = g.tiles_n < tiles_m;
    }
    const int nt = tiles_m * g.tiles_n;
    if ((int)blockIdx.x >= nt * ksplit) return;   // block-uniform (never without the rule)
    const int logical = xcd_logical(blockIdx.x, nt * ksplit);
    const int tile = logical % nt, split = logical / nt;
    const int tm = n_fast ? tile / g.tiles_n : tile % tiles_m;
    const int tn = n_fast ? tile % g.tiles_n : tile / tiles_m;
    const int m0 = tm * BM, n0 = tn * BN;
    const int m_out = g.m_dev ? min(g.m_out, (M + kTokPad - 1) / kTokPad * kTokPad) : g.m_out;
    const int K = g.k_dev ? min(g.K, (*g.k_dev + kTokPad - 1) / kTokPad * kTokPad) : g.K;
    // tiles past the valid rows; an accumulation with an empty K range leaves C as it is
    if (m0 >= (EPI == EPI_DZ ? m_out : M)) return;
    const int kbeg = split * kper;
    const int kend = min(K, kbeg + kper);
    const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
    if (EPI == EPI_ACC && nk == 0 && g.beta) return;

    // Direct-to-LDS loads: one global_load_lds moves 64 lanes x 16 bytes to
    // LDS base + 16*lane, i.e. 8 tile rows of 128 bytes.  Wave w fills rows
    // (4w+q)*8 .. +8 of each operand (q < 4); lane l takes row (l/8) of those
    // and stores k chunk (l%8) ^ swz(row) at LDS position l%8.
    const int lr = lane >> 3, lp = lane & 7;
    int64_t aoff[4];   // element offset of this lane's A rows, -1 past the valid rows
    int arow[4];
    // the epilogue's per-row values are loaded here, so that their latency
    // hides behind the main loop: STATS the target of this lane's result rows
    // (row l%32 of each 32-row block), DZ the per-token factors of row tid
    int ep_y[FM];
    float ep_c2 = 0.0f, ep_cf = 0.0f, ep_ea = 0.0f, ep_eb = 0.0f;
    int ep_yd = -1;
    if (g.a_rows) {
        // independent loads (index clamped; M >= 1 past the exit above), one wait
#pragma unroll
        for (int q = 0; q < 4; ++q) arow[q] = g.a_rows[min(m0 + (wave * 4 + q) * 8 + lr, M - 1)];
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) arow[q] = m0 + (wave * 4 + q) * 8 + lr;
    }
    if constexpr (EPI == EPI_STATS) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = m0 + wm * WM + i * 32 + (lane & 31);
            ep_y[i] = m < M ? g.target[g.a_rows ? g.a_rows[m] : m] : -1;
        }
    } else if constexpr (EPI == EPI_DZ) {
        if (tid < BM) {
            const int m = m0 + tid;
            if (m < M) {
                ep_c2 = g.c2[m];
                ep_cf = g.coef[m];
                if (g.bonus) {
                    ep_ea = g.ea[m];
                    ep_eb = g.eb[m];
                }
                ep_yd = g.target[g.a_rows ? g.a_rows[m] : m];
            }
        }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
        aoff[q] = m0 + (wave * 4 + q) * 8 + lr < M ? (int64_t)arow[q] * g.lda : -1;
    auto issue = [&](int kt) {
        char* st = smem + (kt % NST) * STB;
        const int k0 = kbeg + kt * BK;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = (wave * 4 + q) * 8 + lr;
            const int k = k0 + ((lp ^ swz(r)) << 3);
            const bool kin = k < kend;
            const int nb = n0 + r;
            const uint16_t* ga = (aoff[q] >= 0 && kin) ? g.A + aoff[q] + k : g.zero;
            const uint16_t* gb = (nb < g.N && kin) ? g.B + (int64_t)nb * g.ldb + k : g.zero;
            __builtin_amdgcn_global_load_lds(ga, (lds_void*)(st + (wave * 4 + q) * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(gb, (lds_void*)(st + OPB + (wave * 4 + q) * 1024), 16, 0, 0);
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    const int fr = lane & 31, fh = lane >> 5;
    if (nk > 0) issue(0);
    for (int kt = 0; kt < nk; ++kt) {
        // this wave's loads of stage kt have landed
        __builtin_amdgcn_s_waitcnt(GRPO_VMCNT(0));
        // every wave's share of stage kt is in LDS, and every wave is done
        // reading stage kt-1, which the next issue overwrites
        __syncthreads();
        if (kt + 1 < nk) issue(kt + 1);
        const char* sa = smem + (kt % NST) * STB;
        const char* sb = sa + OPB;
        // the stage's 64 k in two halves of two 16-k MFMA steps each
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            bf16x8 a[2][FM], b[2][FN];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int c = (half * 2 + h) * 2 + fh;   // k chunk: lane half fh holds k = c*8 .. +8
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int r = wm * WM + i * 32 + fr;
                    a[h][i] = *reinterpret_cast<const bf16x8*>(sa + r * ROWB + ((c ^ swz(r)) << 4));
                }
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int r = wn * WN + j * 32 + fr;
                    b[h][j] = *reinterpret_cast<const bf16x8*>(sb + r * ROWB + ((c ^ swz(r)) << 4));
                }
            }
            // all fragment reads of the half before its first MFMA
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[h][i], b[h][j], acc[i][j], 0, 0, 0);
        }
    }

    // result element (i, j, r): row wm*64 + i*32 + (r/4)*8 + (lane/32)*4 + r%4,
    //                           column wn*128 + j*32 + lane%32
    const int rq = fh * 4;
    if constexpr (EPI == EPI_ACC) {
        // per wave, 32 rows of the 64x128 tile at a time go through LDS; then
        // lane l updates column quad l%32 of rows 2k + l/32 with 16-byte
        // accesses (N % 4 == 0 and ldc % 4 == 0, so a quad is all in or all out)
        float* Cs = g.C + (int64_t)split * g.c_split;
        float* T = reinterpret_cast<float*>(smem) + wave * 32 * EPI_ROW_Q;
        const int qc = lane & 31, rh = lane >> 5;
        const int n = n0 + wn * WN + qc * 4;
        __syncthreads();   // the stage buffers are reused
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    T[((r >> 2) * 8 + rq + (r & 3)) * EPI_ROW_Q + j * 32 + fr] = acc[i][j][r];
            __syncthreads();
            if (n < g.N) {
                const int mb = m0 + wm * WM + i * 32 + rh;
                float4 v[16];
#pragma unroll
                for (int k = 0; k < 16; ++k)
                    v[k] = *reinterpret_cast<const float4*>(T + (2 * k + rh) * EPI_ROW_Q + qc * 4);
                if (g.beta) {
                    float4 o[16];
#pragma unroll
                    for (int k = 0; k < 16; ++k)
                        if (mb + 2 * k < M) o[k] = *reinterpret_cast<const float4*>(Cs + (int64_t)(mb + 2 * k) * g.ldc + n);
#pragma unroll
                    for (int k = 0; k < 16; ++k) {
                        v[k].x += o[k].x;
                        v[k].y += o[k].y;
                        v[k].z += o[k].z;
                        v[k].w += o[k].w;
                    }
                }
#pragma unroll
                for (int k = 0; k < 16; ++k)
                    if (mb + 2 * k < M) *reinterpret_cast<float4*>(Cs + (int64_t)(mb + 2 * k) * g.ldc + n) = v[k];
            }
            __syncthreads();
        }
    } else if constexpr (EPI == EPI_DZ) {
        float* s_c2 = reinterpret_cast<float*>(smem);
        float* s_cf = s_c2 + BM;
        float* s_ea = s_cf + BM;
        float* s_eb = s_ea + BM;
        int* s_y = reinterpret_cast<int*>(s_eb + BM);
        char* tcol = smem + DZT_OFF + wave * DZ_WAVEB;   // [column][token] bf16 of this wave, then [token][column]
        uint32_t dpk[FM][FN][4][2] = {};   // the wave's dz values, bf16 pairs (tokens 4q+rq+{0,1}, {2,3})
        __syncthreads();   // the stage buffers are reused
        if (tid < BM) {
            s_c2[tid] = ep_c2;
            s_cf[tid] = ep_cf;
            s_ea[tid] = ep_ea;
            s_eb[tid] = ep_eb;
            s_y[tid] = ep_yd;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int nl = n0 + wn * WN + j * 32 + fr;   // column within the chunk
                if (nl >= g.N) continue;
                const int v = g.col0 + nl;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float d[4];
                    const int mb = wm * WM + i * 32 + q * 8 + rq;   // local row of element r = 4q
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int ml = mb + u;
                        const float cf = s_cf[ml];
                        const float tt = fmaf(acc[i][j][q * 4 + u], kLog2e, -s_c2[ml]);
                        const float pp = __builtin_amdgcn_exp2f(tt);
                        float x;
                        if (!g.bonus) x = cf * pp;
                        else x = pp > 0.0f ? pp * fmaf(s_eb[ml], tt, s_ea[ml]) : 0.0f;
                        if (s_y[ml] == v) x -= cf;
                        d[u] = x;
                    }
                    const int m = m0 + mb;
                    // dz and dz^T go out through LDS: column j*32+fr of the
                    // wave, tokens mb-wm*WM .. +4 (8 bytes)
                    uint2 pk;
                    pk.x = pack2(d[0], d[1]);
                    pk.y = pack2(d[2], d[3]);
                    dpk[i][j][q][0] = pk.x;
                    dpk[i][j][q][1] = pk.y;
                    *reinterpret_cast<uint2*>(tcol + (j * 32 + fr) * DZT_ROWB + (mb - wm * WM) * 2) = pk;
                }
            }
        // each dz^T row segment of the wave (its 64 tokens, 128 bytes) by 8
        // lanes with 16-byte stores; the wave reads only what it wrote
        const int mg = m0 + wm * WM;
        const int64_t koff = g.dzT_off ? *g.dzT_off : 0;
#pragma unroll
        for (int it = 0; it < WN / 8; ++it) {
            const int nloc = it * 8 + (lane >> 3), c = lane & 7;
            const int nl = n0 + wn * WN + nloc;
            const int m = mg + c * 8;
            if (nl < g.N && m < m_out) {
                const char* src = tcol + nloc * DZT_ROWB + c * 16;
                const uint2 lo = *reinterpret_cast<const uint2*>(src);
                const uint2 hi = *reinterpret_cast<const uint2*>(src + 8);
                // non-temporal: dz^T is read by a later GEMM (measured +0.4-0.5 %)
                const u32x4 v4 = {lo.x, lo.y, hi.x, hi.y};
                __builtin_nontemporal_store(v4, reinterpret_cast<u32x4*>(g.dzT + (int64_t)nl * g.ld_dzT + koff + m));
            }
        }
        // then the same buffer as [token][column]: 2-byte writes of the kept
        // values (columns past N were never computed: dpk holds zeros there,
        // and those columns are not stored), then each token row segment of
        // the wave (128 columns, 256 bytes) by 16 lanes with 16-byte stores
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int ml = i * 32 + q * 8 + rq;
                    char* dst = tcol + ml * DZR_ROWB + (j * 32 + fr) * 2;
                    const uint32_t a = dpk[i][j][q][0], b = dpk[i][j][q][1];
                    *reinterpret_cast<uint16_t*>(dst) = (uint16_t)(a & 0xffffu);
                    *reinterpret_cast<uint16_t*>(dst + DZR_ROWB) = (uint16_t)(a >> 16);
                    *reinterpret_cast<uint16_t*>(dst + 2 * DZR_ROWB) = (uint16_t)(b & 0xffffu);
                    *reinterpret_cast<uint16_t*>(dst + 3 * DZR_ROWB) = (uint16_t)(b >> 16);
                }
#pragma unroll
        for (int it = 0; it < 16; ++it) {
            const int ml = it * 4 + (lane >> 4), c = lane & 15;
            const int m = mg + ml;
            const int nl = n0 + wn * WN + c * 8;
            if (m < M && nl < g.N) {
                const char* src = tcol + ml * DZR_ROWB + c * 16;
                const uint2 lo = *reinterpret_cast<const uint2*>(src);
                const uint2 hi = *reinterpret_cast<const uint2*>(src + 8);
                *reinterpret_cast<uint4*>(g.dz + (int64_t)m * g.ld_dz + nl) = make_uint4(lo.x, lo.y, hi.x, hi.y);
            }
        }
    } else {
        // per wave, the 64x128 tile goes through LDS 32 rows at a time; lane l
        // owns row l%32, columns (l/32)*64 .. +64 (rows 528 bytes apart, so the
        // 16 lanes of one 16-byte read pass hit 16 different bank groups)
        float* T = reinterpret_cast<float*>(smem) + wave * 32 * EPI_ROW_Q;
        __syncthreads();   // the stage buffers are reused
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    T[((r >> 2) * 8 + rq + (r & 3)) * EPI_ROW_Q + j * 32 + fr] = acc[i][j][r];
            __syncthreads();
            const int rr = lane & 31, half = lane >> 5;
            const int m = m0 + wm * WM + i * 32 + rr;
            const int nb = n0 + wn * WN + half * 64;
            const int ncols = g.N - nb < 64 ? g.N - nb : 64;
            if (m < M && ncols > 0) {
                const float* row = T + rr * EPI_ROW_Q + half * 64;
                float mx = -INFINITY, se = 0.0f, sw = 0.0f;
                if (ncols == 64) {
                    // the whole slice in registers: 16 reads of 16 bytes, then
                    // the max and the sums in column order
                    float v[64];
#pragma unroll
                    for (int c = 0; c < 16; ++c) {
                        const float4 q = *reinterpret_cast<const float4*>(row + c * 4);
                        v[4 * c] = q.x;
                        v[4 * c + 1] = q.y;
                        v[4 * c + 2] = q.z;
                        v[4 * c + 3] = q.w;
                    }
#pragma unroll
                    for (int c = 0; c < 64; ++c) mx = fmaxf(mx, v[c]);
                    const float cm = mx * kLog2e;
#pragma unroll
                    for (int c = 0; c < 64; ++c) {
                        const float t = fmaf(v[c], kLog2e, -cm);
                        const float e = __builtin_amdgcn_exp2f(t);
                        se += e;
                        sw = fmaf(e, t, sw);
                    }
                } else {
                    for (int c = 0; c < ncols; ++c) mx = fmaxf(mx, row[c]);
                    const float cm = mx * kLog2e;
                    for (int c = 0; c < ncols; ++c) {
                        const float t = fmaf(row[c], kLog2e, -cm);
                        const float e = __builtin_amdgcn_exp2f(t);
                        se += e;
                        sw = fmaf(e, t, sw);
                    }
                }
                g.part[(int64_t)m * g.n_parts + nb / 64] = make_float4(mx, se, sw, 0.0f);
                const int y = ep_y[i];
                if (y >= nb && y < nb + ncols) g.zy[m] = row[y - nb];
            }
            if (g.zst) {
                // z itself, from the same staged rows: lane l writes column
                // quad l%32 of rows 2k + l/32 (two 512-byte row segments per
                // store; N % 4 == 0, so a quad is all in or all out), with
                // the non-temporal hint: z is read back only after the pass
                const int qc = lane & 31, rh = lane >> 5;
                const int n = n0 + wn * WN + qc * 4;
                const int mb = m0 + wm * WM + i * 32 + rh;
                if (n < g.N) {
#pragma unroll
                    for (int k = 0; k < 16; ++k)
                        if (mb + 2 * k < M)
                            __builtin_nontemporal_store(
                                *reinterpret_cast<const f32x4*>(T + (2 * k + rh) * EPI_ROW_Q + qc * 4),
                                reinterpret_cast<f32x4*>(g.zst + (int64_t)(mb + 2 * k) * g.ld_zst + n));
                }
            }
            __syncthreads();
        }
    }
}

// dz of one vocabulary chunk from the stored z (pass 2 without a recompute):
// the dz epilogue's arithmetic on the same fp32 values, so the same bits.
// Block: 64 compact token rows x 128 chunk columns, 256 threads; wave w
// reads rows w*16 + 2k + l/32 (k < 8), column quad l%32, as 512-byte row
// segments.  dz goes out row-major (8-byte stores), dz^T through LDS as
// 128-byte token segments; rows [count, round_up(count, 64)) of dz^T are
// written as zeros (the K padding of the dW GEMM).
struct DzArgs {
    const float* z;        // z[m * ld_z + col0 + c]
    int64_t ld_z;
    int col0, vc;          // chunk start, width (vc % 4 == 0)
    const int32_t* count;  // valid tokens (compact rows)
    const int32_t* vidx;   // token of compact row m
    const int32_t* target;
    const float* c2;
    const float* coef;
    const float* ea;
    const float* eb;
    int bonus;
    uint16_t* dz;          // dz[m * ld_dz + c]
    int64_t ld_dz;
    uint16_t* dzT;         // dzT[c * ld_dzT + koff + m]
    int64_t ld_dzT;
    const int32_t* dzT_off;   // NULL (koff = 0), or the device column offset koff (a dW window's fill)
};

__global__ __launch_bounds__(256) void dz_from_z_kernel(const DzArgs a) {
    constexpr int TR = 64, TC = 128, TROW = TR * 2 + 16;   // dz^T staging: [column][token] bf16, padded rows
    __shared__ __attribute__((aligned(16))) char s_t[TC * TROW];
    __shared__ float s_c2[TR], s_cf[TR], s_ea[TR], s_eb[TR];
    __shared__ int s_y[TR];
    const int cnt = *a.count;
    const int m0 = blockIdx.y * TR, n0 = blockIdx.x * TC;
    if (m0 >= (cnt + kTokPad - 1) / kTokPad * kTokPad) return;   // block-uniform
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (tid < TR) {
        const int m = m0 + tid;
        const bool in = m < cnt;
        s_c2[tid] = in ? a.c2[m] : 0.0f;
        s_cf[tid] = in ? a.coef[m] : 0.0f;
        s_ea[tid] = in && a.bonus ? a.ea[m] : 0.0f;
        s_eb[tid] = in && a.bonus ? a.eb[m] : 0.0f;
        s_y[tid] = in ? a.target[a.vidx[m]] : -1;
    }
    __syncthreads();
    const int qc = lane & 31, rh = lane >> 5;
    const int c = n0 + qc * 4;          // chunk column of this lane's quad
    const bool cin = c < a.vc;
    float4 zv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int ml = wave * 16 + 2 * k + rh, m = m0 + ml;
        // z is read once: a non-temporal load keeps it from displacing what stays
        if (cin && m < cnt) {
            const f32x4 q =
                __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.z + (int64_t)m * a.ld_z + a.col0 + c));
            zv[k] = make_float4(q[0], q[1], q[2], q[3]);
        } else {
            zv[k] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int ml = wave * 16 + 2 * k + rh, m = m0 + ml;
        const float zz[4] = {zv[k].x, zv[k].y, zv[k].z, zv[k].w};
        float d[4];
        const float cf = s_cf[ml], c2 = s_c2[ml];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float tt = fmaf(zz[u], kLog2e, -c2);
            const float pp = __builtin_amdgcn_exp2f(tt);
            float x;
            if (!a.bonus) x = cf * pp;
            else x = pp > 0.0f ? pp * fmaf(s_eb[ml], tt, s_ea[ml]) : 0.0f;
            if (s_y[ml] == a.col0 + c + u) x -= cf;
            d[u] = m < cnt ? x : 0.0f;
        }
        const uint32_t lo = pack2(d[0], d[1]), hi = pack2(d[2], d[3]);
        if (cin && m < cnt) *reinterpret_cast<uint2*>(a.dz + (int64_t)m * a.ld_dz + c) = make_uint2(lo, hi);
        uint16_t* col = reinterpret_cast<uint16_t*>(s_t + (qc * 4) * TROW) + ml;
        col[0] = (uint16_t)(lo & 0xffffu);
        col[TROW / 2] = (uint16_t)(lo >> 16);
        col[TROW] = (uint16_t)(hi & 0xffffu);
        col[3 * TROW / 2] = (uint16_t)(hi >> 16);
    }
    __syncthreads();
    // dz^T: 128 columns x 8 chunks of 16 bytes (8 tokens each)
    const int64_t koff = a.dzT_off ? *a.dzT_off : 0;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int piece = it * 256 + tid, cl = piece >> 3, ch = piece & 7;
        const int cc = n0 + cl;
        if (cc < a.vc)
            // non-temporal: dz^T is read only by the dW GEMM after the chunk's dh
            // (or by the window's flush at the end of the step); dz, read by dh
            // right away, keeps ordinary stores (measured: non-temporal there
            // lost 0.2 %, here it gained 0.5 % of the compaction step)
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(s_t + cl * TROW + ch * 16),
                                        reinterpret_cast<u32x4*>(a.dzT + (int64_t)cc * a.ld_dzT + koff + m0 + ch * 8));
    }
}

// dh row t (H floats) = sum over s, in order, of the partials of t's compact
// row inv[t]; a masked token (inv[t] < 0) gets a zero row.  The split count
// (<= kDhSplitMax): nsplit, or the dh GEMM's rule at the valid-token count
// (rule.cap > 0).  A thread sums four columns of a token, with every split's
// 16-byte load issued before the in-order adds (H % 4 == 0; dst rows 16-byte
// aligned when dst_vec).  Block (x, y): columns [1024x, 1024x + 1024) of
// tokens y, y + gridDim.y, ...
__global__ __launch_bounds__(256) void sum_splits_kernel(float* __restrict__ dst, int64_t ld_dst,
                                                         const float* __restrict__ parts, int nsplit, int64_t c_split,
                                                         const int32_t* __restrict__ inv, int64_t n, int64_t H,
                                                         const int32_t* __restrict__ count, const SplitRule rule,
                                                         int dst_vec) {
    const int64_t c = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (c >= H) return;
    if (rule.cap > 0) nsplit = dev_split_count(rule, *count);
    for (int64_t t = blockIdx.y; t < n; t += gridDim.y) {
        const int32_t j = inv[t];
        float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (j >= 0) {
            const float* p = parts + (int64_t)j * H + c;
            float4 v[kDhSplitMax];
#pragma unroll
            for (int k = 0; k < kDhSplitMax; ++k)
                if (k < nsplit) v[k] = *reinterpret_cast<const float4*>(p + (int64_t)k * c_split);
            s = v[0];
#pragma unroll
            for (int k = 1; k < kDhSplitMax; ++k)
                if (k < nsplit) {
                    s.x += v[k].x;
                    s.y += v[k].y;
                    s.z += v[k].z;
                    s.w += v[k].w;
                }
        }
        float* d = dst + t * ld_dst + c;
        if (dst_vec) {
            *reinterpret_cast<float4*>(d) = s;
        } else {
            d[0] = s.x;
            d[1] = s.y;
            d[2] = s.z;
            d[3] = s.w;
        }
    }
}

// Valid-token compaction of one chunk: vidx[j] = position of the j-th token
// with mask != 0 (in order), inv[t] = its compact index or -1, count[0] = the
// number of valid tokens.  One block, four tokens per thread per pass.
__global__ __launch_bounds__(1024) void compact_tokens_kernel(const uint8_t* __restrict__ mask, int64_t n,
                                                              int32_t* __restrict__ vidx, int32_t* __restrict__ inv,
                                                              int32_t* __restrict__ count) {
    __shared__ int s_wave[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    int base = 0;
    for (int64_t t0 = 0; t0 < n; t0 += 4096) {
        const int64_t t = t0 + (int64_t)tid * 4;
        int v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = (t + u < n && mask[t + u] != 0) ? 1 : 0;
        // valid tokens of the lower lanes of this wave, then of this lane's lower slots
        int pre = 0, mine = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint64_t b = __ballot(v[u]);
            pre += __popcll(b & below);
            mine += __popcll(b);
        }
        if (lane == 0) s_wave[wave] = mine;
        __syncthreads();
        int off = base, tot = 0;
#pragma unroll
        for (int w = 0; w < 16; ++w) {
            off += w < wave ? s_wave[w] : 0;
            tot += s_wave[w];
        }
        int j = off + pre;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (t + u < n) {
                inv[t + u] = v[u] ? j : -1;
                if (v[u]) vidx[j] = (int32_t)(t + u);
            }
            j += v[u];
        }
        base += tot;
        __syncthreads();   // s_wave is rewritten by the next pass
    }
    if (tid == 0) count[0] = base;
}

// One wave per token: merge the token's slice partials in a fixed order,
// then logsumexp, entropy, log-prob, surrogate and gradient coefficient.
struct MergeArgs {
    const float4* part;   // part, zy, c2, coef, ea, eb: at the token's compact index inv[t]
    int n_parts;
    const float* zy;
    const int32_t* inv;
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
    float* c2;
    float* coef;
    float* ea;
    float* eb;
    float* logp;
    float* lse;
    float* entropy;
    float* loss_tok;
    uint8_t* tok_flags;
    grpo_dev::Terms terms;
    float* kl_tok;
};

// (M, S, W): S = sum e^(z-M), W = sum e^(z-M) (z-M) log2(e), merged exactly
__device__ __forceinline__ void merge_part(float& M, float& S, float& W, float m, float s, float w) {
    if (s == 0.0f) return;
    if (S == 0.0f) {
        M = m;
        S = s;
        W = w;
        return;
    }
    const float Mn = fmaxf(M, m);
    const float d1 = (M - Mn) * kLog2e, d2 = (m - Mn) * kLog2e;
    const float f1 = __builtin_amdgcn_exp2f(d1), f2 = __builtin_amdgcn_exp2f(d2);
    const float Sn = S * f1 + s * f2;
    W = f1 * fmaf(S, d1, W) + f2 * fmaf(s, d2, w);
    S = Sn;
    M = Mn;
}

__global__ __launch_bounds__(256) void lm_merge_kernel(const MergeArgs a) {
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (t >= a.n_tok) return;
    const int32_t j = a.inv[t];   // -1 exactly when mask[t] == 0
    if (j < 0) {
        if (lane == 0) {
            if (a.kl_tok) a.kl_tok[t] = 0.0f;
            a.logp[t] = 0.0f;
            if (a.lse) a.lse[t] = 0.0f;
            a.entropy[t] = 0.0f;
            a.loss_tok[t] = 0.0f;
            a.tok_flags[t] = 0;
        }
        return;
    }
    float M = 0.0f, S = 0.0f, W = 0.0f;
    // four slices' loads in flight per lane, merged in the same order as one at a time
    const float4* pp = a.part + (int64_t)j * a.n_parts;
    int p = lane;
    for (; p + 192 < a.n_parts; p += 256) {
        const float4 q0 = pp[p], q1 = pp[p + 64], q2 = pp[p + 128], q3 = pp[p + 192];
        merge_part(M, S, W, q0.x, q0.y, q0.z);
        merge_part(M, S, W, q1.x, q1.y, q1.z);
        merge_part(M, S, W, q2.x, q2.y, q2.z);
        merge_part(M, S, W, q3.x, q3.y, q3.z);
    }
    for (; p < a.n_parts; p += 64) {
        const float4 q = pp[p];
        merge_part(M, S, W, q.x, q.y, q.z);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(M, o), s2 = __shfl_xor(S, o), w2 = __shfl_xor(W, o);
        // the same pair is merged on both lanes; order the operands so both
        // lanes compute bit-identical results
        float Ma = M, Sa = S, Wa = W, Mb = m2, Sb = s2, Wb = w2;
        if ((lane & o) != 0) {
            Ma = m2; Sa = s2; Wa = w2;
            Mb = M; Sb = S; Wb = W;
        }
        merge_part(Ma, Sa, Wa, Mb, Sb, Wb);
        M = Ma;
        S = Sa;
        W = Wa;
    }
    if (lane != 0) return;
    const float log2s = log2f(S);
    const float c2 = M * kLog2e + log2s;
    const float lse = c2 * kLn2;
    const int32_t y = a.target[t];
    const bool ybad = (uint32_t)y >= (uint64_t)a.V;
    const float logp = ybad ? __builtin_nanf("") : a.zy[j] - lse;
    const float H = kLn2 * (log2s - W / S);
    const int32_t row = a.tok_row[t];
    const float A = ((uint32_t)row < (uint64_t)a.n_rows) ? a.adv_row[row] : __builtin_nanf("");
    const float sf = grpo_dev::token_factor(grpo_dev::step_scale(a.scale, a.denom), a.terms.row_weight, row,
                                            a.n_rows);
    const grpo_dev::Surrogate sg = grpo_dev::surrogate(logp, H, a.old_logp[t], A, a.eps_low, a.eps_high, sf,
                                                       a.terms, t);
    const float e = a.terms.ent_coef * sf;
    a.c2[j] = c2;
    a.coef[j] = sg.coef;
    a.ea[j] = fmaf(e, H, sg.coef);
    a.eb[j] = e * kLn2;
    if (a.kl_tok) a.kl_tok[t] = sg.kl;
    a.logp[t] = logp;
    if (a.lse) a.lse[t] = lse;
    a.entropy[t] = H;
    a.loss_tok[t] = sg.loss;
    a.tok_flags[t] = (uint8_t)(1u | (sg.clipped ? 2u : 0u) | (sg.bad ? 4u : 0u));
}

// dst[c * ld_dst + off + r] = src[row(r) * ld_src + c] for r < rows, c < cols,
// with row(r) = rmap ? rmap[r] : r and rows = min(rows, *rcount) when rcount
// is set; columns [rows, rows_pad) of dst are written as zeros.  With dst_off
// (a dW window's device fill), off = *dst_off and rows_pad is cut to rows
// rounded up to 64, so that the window's next call starts there.  64x64
// tiles through LDS, moved as pieces of eight elements: 16-byte loads and
// stores when vec (src and dst 16-byte aligned, ld_src and ld_dst multiples
// of 8), element by element otherwise and at the edges.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ src, int64_t rows,
                                                             int64_t cols, int64_t ld_src, uint16_t* __restrict__ dst,
                                                             int64_t ld_dst, int64_t rows_pad,
                                                             const int32_t* __restrict__ rmap,
                                                             const int32_t* __restrict__ rcount,
                                                             const int32_t* __restrict__ dst_off, int vec) {
    // tile[r][c]: 64 source rows of 64 columns, rows 144 bytes apart (16-byte pieces stay aligned)
    __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];
    const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
    const int tid = threadIdx.x;
    if (rcount && *rcount < rows) rows = *rcount;
    if (dst_off) {
        dst += *dst_off;
        const int64_t rp = (rows + 63) / 64 * 64;
        if (rp < rows_pad) rows_pad = rp;
    }
    if (r0 >= rows_pad) return;   // block-uniform
    // in: piece i of 512 is source row i/8, columns (i%8)*8 .. +8 (zeros past rows and cols)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int i = h * 256 + tid, r = i >> 3, cc = (i & 7) * 8;
        const int64_t gr = r0 + r, gc = c0 + cc;
        uint4 q = make_uint4(0u, 0u, 0u, 0u);
        if (gr < rows) {
            const uint16_t* sp = src + (rmap ? (int64_t)rmap[gr] : gr) * ld_src + gc;
            if (vec && gc + 8 <= cols) {
                q = *reinterpret_cast<const uint4*>(sp);
            } else {
                uint32_t w[4] = {0u, 0u, 0u, 0u};
                for (int e = 0; e < 8; ++e)
                    if (gc + e < cols) w[e >> 1] |= (uint32_t)sp[e] << ((e & 1) * 16);
                q = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
        *reinterpret_cast<uint4*>(&tile[r][cc]) = q;
    }
    __syncthreads();
    // out: piece i of 512 is destination row (source column) i/8, tokens (i%8)*8 .. +8
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int i = h * 256 + tid, c = i >> 3, rr = (i & 7) * 8;
        const int64_t gc = c0 + c, gr = r0 + rr;
        if (gc >= cols || gr >= rows_pad) continue;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (uint32_t)tile[rr + 2 * e][c] | ((uint32_t)tile[rr + 2 * e + 1][c] << 16);
        uint16_t* dp = dst + gc * ld_dst + gr;
        if (vec && gr + 8 <= rows_pad) {
            *reinterpret_cast<uint4*>(dp) = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
            for (int e = 0; e < 8; ++e)
                if (gr + e < rows_pad) dp[e] = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
        }
    }
}

// A dW window's fill counter: advanced by the chunk's valid tokens rounded up
// to 64 (count non-NULL), or cleared (count NULL).  Runs after every kernel
// of the chunk that reads the counter.
__global__ void dw_fill_kernel(int32_t* fill, const int32_t* count) {
    if (threadIdx.x == 0) *fill = count ? *fill + (*count + kTokPad - 1) / kTokPad * kTokPad : 0;
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// A dW window's buffer: the fill counter (columns written so far, a multiple
// of 64), h^T [H x cap] and dz^T [V x cap], cap = cap_tok rounded up to 64.
struct WindowLayout {
    int32_t* fill;
    uint16_t* hT;
    uint16_t* dzT;
    int64_t cap;
    size_t bytes;
};

WindowLayout window_layout(void* buf, int64_t cap_tok, int64_t H, int64_t V) {
    WindowLayout l{};
    l.cap = round_up(cap_tok, kTokPad);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = (size_t)round_up((int64_t)(off + bytes), 256);
        return reinterpret_cast<char*>(buf) + at;
    };
    l.fill = reinterpret_cast<int32_t*>(take(4));
    l.hT = reinterpret_cast<uint16_t*>(take((size_t)H * l.cap * 2));
    l.dzT = reinterpret_cast<uint16_t*>(take((size_t)V * l.cap * 2));
    l.bytes = off;
    return l;
}

bool window_sizes_ok(int64_t cap_tok, int64_t H, int64_t V) {
    return cap_tok >= 1 && cap_tok <= (1LL << 30) && H > 0 && V > 0 && H % 8 == 0 && V % 8 == 0 && V <= (1 << 30) &&
           H <= (1 << 20);
}

struct Workspace {
    float4* part;
    float* zy;
    float* c2;
    float* coef;
    float* ea;
    float* eb;
    uint16_t* hT;
    float* z;         // pass 1's z of the valid tokens [n x V] (NULL: pass 2 recomputes it)
    uint16_t* dz;
    uint16_t* dzT;
    float* dh_part;
    int32_t* vidx;    // valid-token compaction of the chunk
    int32_t* inv;
    int32_t* count;   // number of valid tokens
    size_t bytes;
};

// Pass 2 plan.  Every block of these GEMMs fills one compute unit, so a
// launch of b blocks costs ceil(b / CUs) rounds of its per-block k-steps.
// The vocabulary chunk width (a multiple of the tile width, at most
// kVocabChunkMax) and the split count of dh = dz W_c (its output has only
// ceil(n/256) x ceil(H/256) tiles, so its K range, the chunk's vocabulary, is
// split; one partial per split, the same count for every chunk) are chosen
// to minimise the summed rounds x k-steps of the dz, dh and dW launches plus
// the HBM time of the dh partials: each split's n x H fp32 partial is written
// by the first chunk, read and rewritten by every later one and read once by
// the final sum (2 x chunks x splits partials moved), converted to k-step
// units with the measured rates (a 256 x 256 x 64 block step takes ~2 us at
// ~1 PFLOP/s; HBM moves ~5 bytes per ns).
struct Pass2Plan {
    int64_t chunk;
    int nsplit;
    double cost;
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// chunk_cap (a multiple of BN) and split_cap bound the plan to a smaller
// workspace (the no-allocation entry point's fixed scratch).
Pass2Plan plan_pass2(int64_t n, int64_t H, int64_t V, int64_t cus, int64_t chunk_cap = kVocabChunkMax,
                     int split_cap = kDhSplitMax, bool stash = false, bool defer = false) {
    const int64_t n_pad = round_up(n, kTokPad);
    const int64_t tm = cdiv(n, BM), th = cdiv(H, BN);
    const int64_t wcap = chunk_cap;
    Pass2Plan best{V < wcap ? V : wcap, 1, -1.0};
    double best_cost = -1.0;
    const int64_t wmax = V < wcap ? round_up(V, BN) : wcap;
    // with the logits kept, one chunk over all of V: one dh launch per call and
    // partials written once, not rewritten (measured 0.4-0.9 % on the step)
    const int64_t wmin = stash ? wmax : (wmax < kVocabChunkMin ? wmax : kVocabChunkMin);
    for (int64_t w = wmin; w <= wmax; w += 2048 > wmax - wmin ? BN : 2048) {
        for (int sp = 1; sp <= split_cap; ++sp) {
            int64_t steps = 0, chunks = 0;
            for (int64_t c0 = 0; c0 < V; c0 += w) {
                const int64_t vc = V - c0 < w ? V - c0 : w, tv = cdiv(vc, BN);
                if (!stash) steps += cdiv(tm * tv, cus) * cdiv(H, BK);                  // dz (recomputed)
                if (!defer) steps += cdiv(tv * th, cus) * cdiv(n_pad, BK);              // dW
                steps += cdiv(tm * th * sp, cus) * (round_up(cdiv(vc, sp), BK) / BK);   // dh
                ++chunks;
            }
            const double partial_bytes = 2.0 * (double)chunks * sp * (double)n * (double)H * 4.0;
            const double cost = (double)steps + partial_bytes / (kHbmBytesPerUs * kKstepUs);
            // a split must save at least 1 % to be worth its partial
            if (best_cost < 0.0 || cost * 100.0 < best_cost * 99.0) {
                best_cost = cost;
                best = {w < V ? w : V, sp, cost};
            }
        }
    }
    return best;
}

Workspace carve(void* base, int64_t n_tok, int64_t H, int64_t V, int64_t chunk_cap = kVocabChunkMax,
                int split_cap = kDhSplitMax, bool stash = false, bool defer = false) {
    const int64_t n_parts = (V + 63) / 64;
    const int64_t n_pad = round_up(n_tok > 0 ? n_tok : 1, kTokPad);
    const int64_t vc = V < chunk_cap ? V : chunk_cap;   // widest chunk any plan within the caps uses
    Workspace w{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = (size_t)round_up((int64_t)(off + bytes), 256);
        return reinterpret_cast<char*>(base) + at;
    };
    w.part = reinterpret_cast<float4*>(take((size_t)n_tok * n_parts * sizeof(float4)));
    w.zy = reinterpret_cast<float*>(take((size_t)n_tok * 4));
    w.c2 = reinterpret_cast<float*>(take((size_t)n_tok * 4));
    w.coef = reinterpret_cast<float*>(take((size_t)n_tok * 4));
    w.ea = reinterpret_cast<float*>(take((size_t)n_tok * 4));
    w.eb = reinterpret_cast<float*>(take((size_t)n_tok * 4));
    // with a dW window, h^T and dz^T go there
    w.hT = defer ? nullptr : reinterpret_cast<uint16_t*>(take((size_t)H * n_pad * 2));
    w.z = stash ? reinterpret_cast<float*>(take((size_t)n_tok * V * 4)) : nullptr;
    w.dz = reinterpret_cast<uint16_t*>(take((size_t)n_tok * vc * 2));
    w.dzT = defer ? nullptr : reinterpret_cast<uint16_t*>(take((size_t)vc * n_pad * 2));
    w.dh_part = reinterpret_cast<float*>(take((size_t)split_cap * n_tok * H * 4));
    w.vidx = reinterpret_cast<int32_t*>(take((size_t)n_tok * 4));
    w.inv = reinterpret_cast<int32_t*>(take((size_t)n_tok * 4));
    w.count = reinterpret_cast<int32_t*>(take(4));
    w.bytes = off;
    return w;
}

template <int EPI>
hipError_t launch_gemm(GemmArgs g, hipStream_t st) {
    g.tiles_m = (g.M + BM - 1) / BM;
    g.tiles_n = (g.N + BN - 1) / BN;
    if (EPI == EPI_DZ) g.tiles_m = (g.m_out + BM - 1) / BM;
    // the index with fewer tiles varies fastest, so the blocks that read one
    // tile of the larger operand are adjacent and share it in L2
    g.n_fast = g.tiles_n < g.tiles_m;
    if (g.ksplit < 1) {
        g.ksplit = 1;
        g.kper = g.K;
    }
    const long long nb = (long long)g.tiles_m * g.tiles_n * g.ksplit;
    if (nb == 0) return hipSuccess;
    // the zero page's address as an argument: taken from the symbol in the
    // loop, it was reloaded from memory after every barrier
    hipError_t e = hipGetSymbolAddress((void**)&g.zero, HIP_SYMBOL(g_zero_page));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gemm_nt_kernel<EPI>, dim3((unsigned)nb), dim3(NTHREADS), 0, st, g);
    return hipGetLastError();
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int dev_fail(hipError_t e, const char* what) {
    return fail(GRPO_EDEVICE, "grpo_lmhead_fwd_bwd (%s): %s", what, hipGetErrorString(e));
}

// With GRPO_LMHEAD_KEEP_Z pass 1 keeps z (fp32) and pass 2 reads it back
// instead of recomputing it; the vocabulary chunk may then span all of V.
int64_t stash_chunk_cap(int64_t V) { return round_up(V, BN); }

}  // namespace

extern "C" size_t grpo_lmhead_workspace_size_flags(int64_t n_tok, int64_t H, int64_t V, int32_t flags) {
    if (n_tok < 0 || H <= 0 || V <= 0 || (flags & ~(GRPO_LMHEAD_KEEP_Z | GRPO_LMHEAD_DEFER_DW))) return 0;
    const bool stash = (flags & GRPO_LMHEAD_KEEP_Z) != 0, defer = (flags & GRPO_LMHEAD_DEFER_DW) != 0;
    return carve(nullptr, n_tok, H, V, (stash || defer) ? stash_chunk_cap(V) : kVocabChunkMax, kDhSplitMax, stash,
                 defer).bytes;
}

namespace {

// A window as set up by grpo_lmhead_dw_window_init and kept by the calls.
int check_window(const char* who, const grpo_lmhead_dw_window* w) {
    if (!w || !w->buf || (reinterpret_cast<uintptr_t>(w->buf) & 255u) || !window_sizes_ok(w->cap_tok, w->H, w->V))
        return fail(GRPO_EINVAL, "%s: dW window missing or not set up (grpo_lmhead_dw_window_init)", who);
    const WindowLayout l = window_layout(nullptr, w->cap_tok, w->H, w->V);
    if (w->bytes < l.bytes || w->reserved < 0 || w->reserved > l.cap || w->reserved % kTokPad)
        return fail(GRPO_EINVAL, "%s: dW window fields changed since grpo_lmhead_dw_window_init", who);
    return GRPO_OK;
}

}  // namespace

extern "C" size_t grpo_lmhead_dw_window_size(int64_t cap_tok, int64_t H, int64_t V) {
    return window_sizes_ok(cap_tok, H, V) ? window_layout(nullptr, cap_tok, H, V).bytes : 0;
}

extern "C" int grpo_lmhead_dw_window_init(void* stream, grpo_lmhead_dw_window* w, void* buf, size_t bytes,
                                          int64_t cap_tok, int64_t H, int64_t V) {
    if (!w || !buf || (reinterpret_cast<uintptr_t>(buf) & 255u) || !window_sizes_ok(cap_tok, H, V))
        return fail(GRPO_EINVAL, "grpo_lmhead_dw_window_init: need w, a 256-byte aligned buf, 1 <= cap_tok <= 2^30, "
                    "H and V positive multiples of 8");
    const WindowLayout l = window_layout(buf, cap_tok, H, V);
    if (bytes < l.bytes)
        return fail(GRPO_ECAPACITY, "grpo_lmhead_dw_window_init: %zu bytes needed for %lld tokens", l.bytes,
                    (long long)cap_tok);
    hipLaunchKernelGGL(dw_fill_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, l.fill, nullptr);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(GRPO_EDEVICE, "grpo_lmhead_dw_window_init: %s", hipGetErrorString(e));
    *w = grpo_lmhead_dw_window{buf, bytes, cap_tok, H, V, 0};
    return ok();
}

extern "C" int grpo_lmhead_dw_flush(void* stream, grpo_lmhead_dw_window* w, float* dW) {
    int rc = check_window("grpo_lmhead_dw_flush", w);
    if (rc != GRPO_OK) return rc;
    if (!dW || !al16(dW)) return fail(GRPO_EINVAL, "grpo_lmhead_dw_flush: dW is required (16-byte aligned)");
    if (w->reserved == 0) return ok();
    const WindowLayout l = window_layout(w->buf, w->cap_tok, w->H, w->V);
    hipStream_t st = (hipStream_t)stream;
    // dW += dz^T h over the window's columns: K bounded by the reserved
    // columns on the host, by the fill counter (the valid tokens) in the kernel
    GemmArgs gw{};
    gw.A = l.dzT; gw.lda = l.cap; gw.B = l.hT; gw.ldb = l.cap;
    gw.M = (int)w->V; gw.N = (int)w->H; gw.K = (int)w->reserved;
    gw.k_dev = l.fill;
    gw.C = dW; gw.ldc = w->H; gw.beta = 1;
    hipError_t e = launch_gemm<EPI_ACC>(gw, st);
    if (e == hipSuccess) {
        hipLaunchKernelGGL(dw_fill_kernel, dim3(1), dim3(64), 0, st, l.fill, nullptr);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return fail(GRPO_EDEVICE, "grpo_lmhead_dw_flush: %s", hipGetErrorString(e));
    w->reserved = 0;
    return ok();
}

extern "C" size_t grpo_lmhead_workspace_size(int64_t n_tok, int64_t H, int64_t V) {
    return grpo_lmhead_workspace_size_flags(n_tok, H, V, 0);
}

extern "C" int grpo_transpose_bf16(void* stream, const void* src, int64_t rows, int64_t cols, int64_t ld_src,
                                   void* dst, int64_t ld_dst) {
    if (rows < 0 || cols < 0 || ld_src < cols || ld_dst < rows || (rows > 0 && cols > 0 && (!src || !dst)))
        return fail(GRPO_EINVAL, "grpo_transpose_bf16: bad arguments");
    if (rows == 0 || cols == 0) return ok();
    if ((rows + 63) / 64 > 65535 || (cols + 63) / 64 > 0x7fffffffLL)
        return fail(GRPO_EINVAL, "grpo_transpose_bf16: too many rows for one launch");
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64)),
                       dim3(256), 0, (hipStream_t)stream, (const uint16_t*)src, rows, cols, ld_src, (uint16_t*)dst,
                       ld_dst, rows, nullptr, nullptr, nullptr, (int)(al16(src) && al16(dst) && ld_src % 8 == 0 &&
                                                                      ld_dst % 8 == 0));
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? ok() : fail(GRPO_EDEVICE, "grpo_transpose_bf16: %s", hipGetErrorString(e));
}

namespace {

// The scratch of grpo_lmhead_fwd_bwd_noalloc: one array per device, held by
// the loaded library until the process ends.  On the host `scratch` names a
// stand-in, not device memory: kernels get the address from
// hipGetSymbolAddress, taken once per device (scratch_ptr).
constexpr size_t kStaticScratchBytes = (size_t)GRPO_LMHEAD_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up once per
// device, with that device current).
int scratch_ptr(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GRPO_EDEVICE, "grpo_lmhead_fwd_bwd_noalloc: hipGetDevice: %s",
                                     hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(GRPO_EDEVICE, "grpo_lmhead_fwd_bwd_noalloc: device %d beyond the %d the library tracks", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(GRPO_EDEVICE, "grpo_lmhead_fwd_bwd_noalloc: hipGetSymbolAddress(scratch): %s",
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GRPO_OK;
}

// Caps (vocabulary chunk width, dh splits) whose workspace fits `cap` bytes,
// the cheapest such plan by plan_pass2's cost; chunk 0 when none fits.
Pass2Plan plan_within(int64_t n, int64_t H, int64_t V, int64_t cus, size_t cap, int64_t* chunk_cap,
                      int* split_cap) {
    Pass2Plan best{0, 0, -1.0};
    *chunk_cap = 0;
    *split_cap = 0;
    for (int sp = kDhSplitMax; sp >= 1; sp = sp > 1 ? sp / 2 : 0) {
        // the widest chunk (a multiple of BN) whose workspace fits, by bisection
        int64_t lo = 0, hi = kVocabChunkMax / BN;
        while (lo < hi) {
            const int64_t mid = (lo + hi + 1) / 2;
            if (carve(nullptr, n, H, V, mid * BN, sp).bytes <= cap) lo = mid;
            else hi = mid - 1;
        }
        if (lo == 0) continue;
        const Pass2Plan p = plan_pass2(n, H, V, cus, lo * BN, sp);
        if (best.cost < 0.0 || p.cost < best.cost) {
            best = p;
            *chunk_cap = lo * BN;
            *split_cap = sp;
        }
    }
    return best;
}

int lmhead_run(void* stream, const grpo_lmhead_args* a, bool noalloc);

}  // namespace

extern "C" int grpo_lmhead_fwd_bwd(void* stream, const grpo_lmhead_args* a) {
    return lmhead_run(stream, a, false);
}

extern "C" int grpo_lmhead_fwd_bwd_noalloc(void* stream, const grpo_lmhead_args* a) {
    return lmhead_run(stream, a, true);
}

namespace {

int lmhead_run(void* stream, const grpo_lmhead_args* a, bool noalloc) {
    if (!a) return fail(GRPO_EINVAL, "grpo_lmhead_fwd_bwd: NULL args");
    if (a->struct_size != (int32_t)sizeof(grpo_lmhead_args))
        return fail(GRPO_EINVAL, "grpo_lmhead_fwd_bwd: struct_size %d != %d", a->struct_size,
                    (int)sizeof(grpo_lmhead_args));
    const int64_t n = a->n_tok, H = a->H, V = a->V;
    if (n < 0 || H <= 0 || V <= 0 || a->n_rows < 0 || (n > 0 && a->n_rows < 1))
        return fail(GRPO_EINVAL, "grpo_lmhead_fwd_bwd: need n_tok >= 0, H > 0, V > 0, rows for the tokens");
    if (H % 8 || V % 8 || a->ldh < H || a->ldh % 8)
        return fail(GRPO_EINVAL, "grpo_lmhead_fwd_bwd: H, V and ldh must be multiples of 8 (ldh >= H)");
    if (n > kMaxTokens || V > (1 << 30) || H > (1 << 20))
        return fail(GRPO_EINVAL, "grpo_lmhead_fwd_bwd: n_tok above %lld or sizes beyond the kernels' 32-bit tile "
                    "indexing", (long long)kMaxTokens);
    const bool defer = (a->flags & GRPO_LMHEAD_DEFER_DW) != 0;
    if (!a->W || !a->Wt || (!defer && !a->dW) || !al16(a->W) || !al16(a->Wt) || !al16(a->dW))
        return fail(GRPO_EINVAL, "grpo_lmhead_fwd_bwd: W, Wt and dW (unless deferred) are required (16-byte aligned)");
    if (!a->chunk_stats || (a->n_rows > 0 && (!a->row_stats || !a->row_off)))
        return fail(GRPO_EINVAL, "grpo_lmhead_fwd_bwd: NULL stats pointer");
    if (n > 0 && (!a->h || !al16(a->h) || !a->target || !a->mask || !a->old_logp || !a->tok_row || !a->adv_row ||
                  !a->dh || !a->logp || !a->entropy || !a->loss_tok || !a->tok_flags))
        return fail(GRPO_EINVAL, "grpo_lmhead_fwd_bwd: NULL or misaligned pointer");
    if (!(a->eps_low >= 0.0f && a->eps_low <= 1.0f && a->eps_high >= 0.0f && std::isfinite(a->eps_high)) ||
        !std::isfinite(a->scale))
        return fail(GRPO_EINVAL, "grpo_lmhead_fwd_bwd: bad clip band or scale");
    {
        const int rc = grpo::check_terms("grpo_lmhead_fwd_bwd", n, a->ref_logp, a->kl_tok, a->ent_coef, a->kl_coef,
                                         a->kl_type);
        if (rc != GRPO_OK) return rc;
    }
    if (a->flags & ~(GRPO_LMHEAD_KEEP_Z | GRPO_LMHEAD_DEFER_DW))
        return fail(GRPO_EINVAL, "grpo_lmhead_fwd_bwd: unknown flags %d", a->flags);
    const bool stash = (a->flags & GRPO_LMHEAD_KEEP_Z) != 0;
    if (stash && noalloc)
        return fail(GRPO_EINVAL, "grpo_lmhead_fwd_bwd_noalloc: GRPO_LMHEAD_KEEP_Z needs a caller workspace (the "
                    "chunk's logits do not fit the fixed scratch)");
    if (defer && noalloc)
        return fail(GRPO_EINVAL, "grpo_lmhead_fwd_bwd_noalloc: GRPO_LMHEAD_DEFER_DW belongs to the workspace path");
    grpo_lmhead_dw_window* win = a->dw_window;
    if (defer != (win != nullptr))
        return fail(GRPO_EINVAL, "grpo_lmhead_fwd_bwd: GRPO_LMHEAD_DEFER_DW and dw_window go together");
    const int64_t reserve = defer ? round_up(n, kTokPad) : 0;
    if (defer) {
        const int rc = check_window("grpo_lmhead_fwd_bwd", win);
        if (rc != GRPO_OK) return rc;
        if (win->H != H || win->V != V)
            return fail(GRPO_EINVAL, "grpo_lmhead_fwd_bwd: the dW window is for H %lld, V %lld", (long long)win->H,
                        (long long)win->V);
        if (win->reserved + reserve > round_up(win->cap_tok, kTokPad))
            return fail(GRPO_ECAPACITY, "grpo_lmhead_fwd_bwd: the dW window has %lld of %lld columns reserved and "
                        "this chunk needs %lld more; flush it first", (long long)win->reserved,
                        (long long)round_up(win->cap_tok, kTokPad), (long long)reserve);
    }
    int dev = 0, cus = 0;
    hipError_t e;
    if ((e = hipGetDevice(&dev)) != hipSuccess ||
        (e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
        return dev_fail(e, "device query");
    if (cus < 1) cus = 1;
    void* wsp = a->workspace;
    int64_t chunk_cap = kVocabChunkMax;
    int split_cap = kDhSplitMax;
    Pass2Plan plan{};
    if (noalloc) {
        // the library's own scratch; the caller's workspace fields are ignored
        plan = plan_within(n, H, V, cus, kStaticScratchBytes, &chunk_cap, &split_cap);
        if (chunk_cap == 0)
            return fail(GRPO_ECAPACITY, "grpo_lmhead_fwd_bwd_noalloc: %lld tokens at H %lld, V %lld need %zu bytes of "
                        "scratch even with the narrowest plan; the fixed scratch holds %zu",
                        (long long)n, (long long)H, (long long)V, carve(nullptr, n, H, V, BN, 1).bytes,
                        kStaticScratchBytes);
        const int rc = scratch_ptr(&wsp);
        if (rc != GRPO_OK) return rc;
    } else {
        const size_t need = grpo_lmhead_workspace_size_flags(n, H, V, a->flags);
        if (!a->workspace || a->workspace_bytes < need || !al16(a->workspace))
            return fail(GRPO_ECAPACITY, "grpo_lmhead_fwd_bwd: workspace of %zu bytes needed (16-byte aligned)", need);
        // with the logits kept or dz^T in a window the workspace holds no dz^T
        // chunk, and the chunk may span all of V (measured +0.9 % on the step with
        // the window alone; the plan still chooses the width)
        if (stash || defer) chunk_cap = stash_chunk_cap(V);
        plan = plan_pass2(n, H, V, cus, chunk_cap, split_cap, stash, defer);
    }
    hipStream_t st = (hipStream_t)stream;
    const grpo::ObjTerms obj{a->scale, a->denom, a->row_weight, a->ent_coef, a->ref_logp ? a->kl_coef : 0.0f};
    float* kl_tok = a->ref_logp ? a->kl_tok : nullptr;
    if (n == 0) return grpo::launch_stats(stream, a->loss_tok, a->entropy, kl_tok, a->tok_flags, a->row_off,
                                          a->n_rows, 0, obj, a->row_stats, a->chunk_stats);
    const Workspace w = carve(wsp, n, H, V, chunk_cap, split_cap, stash, defer);
    // with a dW window, h^T and dz^T of the valid tokens are appended to it at
    // its fill counter; else they live in the workspace
    const WindowLayout wl = defer ? window_layout(win->buf, win->cap_tok, H, V) : WindowLayout{};
    uint16_t* const hT = defer ? wl.hT : w.hT;
    const int64_t ld_T = defer ? wl.cap : round_up(n, kTokPad);
    const int32_t* const fill = defer ? wl.fill : nullptr;
    const int64_t n_pad = round_up(n, kTokPad);
    const int n_parts = (int)((V + 63) / 64);
    const uint16_t* h = (const uint16_t*)a->h;
    const uint16_t* W = (const uint16_t*)a->W;
    const uint16_t* Wt = (const uint16_t*)a->Wt;

    // Masked tokens add nothing to any product (their dz rows are zero), so
    // the GEMMs run over the chunk's valid tokens only: vidx lists them in
    // order, inv maps a token to its compact index, count holds how many.
    // Grids stay sized for all n tokens; the kernels read the count.
    hipLaunchKernelGGL(compact_tokens_kernel, dim3(1), dim3(1024), 0, st, a->mask, n, w.vidx, w.inv, w.count);
    if ((e = hipGetLastError()) != hipSuccess) return dev_fail(e, "compaction");

    // h^T of the valid tokens, zero columns up to n_pad (the K operand of dW's GEMM)
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)((H + 63) / 64), (unsigned)((n_pad + 63) / 64)),
                       dim3(256), 0, st, h, n, H, a->ldh, hT, ld_T, n_pad, w.vidx, w.count, fill,
                       (int)(al16(h) && al16(hT) && a->ldh % 8 == 0 && ld_T % 8 == 0));
    if ((e = hipGetLastError()) != hipSuccess) return dev_fail(e, "transpose h");

    // pass 1: slice partials of the log-softmax and the target logit
    GemmArgs g{};
    g.A = h; g.lda = a->ldh; g.B = W; g.ldb = H;
    g.M = (int)n; g.N = (int)V; g.K = (int)H;
    g.a_rows = w.vidx; g.m_dev = w.count;
    g.part = w.part; g.n_parts = n_parts; g.target = a->target; g.zy = w.zy;
    g.zst = w.z; g.ld_zst = V;
    if ((e = launch_gemm<EPI_STATS>(g, st)) != hipSuccess) return dev_fail(e, "pass 1");

    MergeArgs mg{};
    mg.part = w.part; mg.n_parts = n_parts; mg.zy = w.zy; mg.inv = w.inv; mg.n_tok = n; mg.V = V;
    mg.target = a->target; mg.mask = a->mask; mg.old_logp = a->old_logp; mg.tok_row = a->tok_row;
    mg.adv_row = a->adv_row; mg.n_rows = a->n_rows; mg.eps_low = a->eps_low; mg.eps_high = a->eps_high;
    mg.scale = a->scale; mg.denom = a->denom; mg.c2 = w.c2; mg.coef = w.coef; mg.ea = w.ea; mg.eb = w.eb;
    mg.logp = a->logp; mg.lse = a->lse;
    mg.terms = grpo_dev::Terms{a->row_weight, a->ref_logp, a->ent_coef, a->kl_coef, a->kl_type};
    mg.kl_tok = kl_tok;
    mg.entropy = a->entropy; mg.loss_tok = a->loss_tok; mg.tok_flags = a->tok_flags;
    hipLaunchKernelGGL(lm_merge_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, st, mg);
    if ((e = hipGetLastError()) != hipSuccess) return dev_fail(e, "merge");
    const int rc = grpo::launch_stats(stream, a->loss_tok, a->entropy, kl_tok, a->tok_flags, a->row_off, a->n_rows,
                                      n, obj, a->row_stats, a->chunk_stats);
    if (rc != GRPO_OK) return rc;

    // pass 2: per vocabulary chunk, dz then dh (+)= dz W_c and dW_c += dz^T h
    const int64_t chunk = plan.chunk;
    const int nsplit = plan.nsplit;
    // dh's split count follows the valid rows, on the device (SplitRule)
    const SplitRule rule{split_cap, (int)chunk, (int)cdiv(V, chunk), cus, (int)cdiv(H, BN), (int)H};
    for (int64_t c0 = 0; c0 < V; c0 += chunk) {
        const int vc = (int)(V - c0 < chunk ? V - c0 : chunk);
        if (stash) {
            DzArgs d{};
            d.z = w.z; d.ld_z = V; d.col0 = (int)c0; d.vc = vc;
            d.count = w.count; d.vidx = w.vidx; d.target = a->target;
            d.c2 = w.c2; d.coef = w.coef; d.ea = w.ea; d.eb = w.eb; d.bonus = a->ent_coef != 0.0f;
            d.dz = w.dz; d.ld_dz = vc; d.dzT = defer ? wl.dzT + c0 * wl.cap : w.dzT; d.ld_dzT = ld_T;
            d.dzT_off = fill;
            hipLaunchKernelGGL(dz_from_z_kernel, dim3((unsigned)((vc + 127) / 128), (unsigned)(n_pad / 64)),
                               dim3(256), 0, st, d);
            if ((e = hipGetLastError()) != hipSuccess) return dev_fail(e, "dz");
        } else {
            GemmArgs d{};
            d.A = h; d.lda = a->ldh; d.B = W + c0 * H; d.ldb = H;
            d.M = (int)n; d.N = vc; d.K = (int)H;
            d.a_rows = w.vidx; d.m_dev = w.count;
            d.c2 = w.c2; d.coef = w.coef; d.target = a->target; d.col0 = (int)c0; d.m_out = (int)n_pad;
            d.ea = w.ea; d.eb = w.eb; d.bonus = a->ent_coef != 0.0f;
            d.dz = w.dz; d.ld_dz = vc; d.dzT = defer ? wl.dzT + c0 * wl.cap : w.dzT; d.ld_dzT = ld_T;
            d.dzT_off = fill;
            if ((e = launch_gemm<EPI_DZ>(d, st)) != hipSuccess) return dev_fail(e, "dz");
        }

        // dh: the chunk's vocabulary range split nsplit ways, split s
        // accumulating into its own partial (summed in order at the end)
        GemmArgs gh{};
        gh.A = w.dz; gh.lda = vc; gh.B = Wt + c0; gh.ldb = V;
        gh.M = (int)n; gh.N = (int)H; gh.K = vc;
        gh.m_dev = w.count;
        gh.split = rule;
        gh.ksplit = rule.cap;
        gh.kper = (int)round_up(vc, BK);
        gh.C = w.dh_part; gh.ldc = H; gh.c_split = n * H; gh.beta = c0 > 0;
        if ((e = launch_gemm<EPI_ACC>(gh, st)) != hipSuccess) return dev_fail(e, "dh");

        if (!defer) {
            GemmArgs gw{};
            gw.A = w.dzT; gw.lda = n_pad; gw.B = w.hT; gw.ldb = n_pad;
            gw.M = vc; gw.N = (int)H; gw.K = (int)n_pad;
            gw.k_dev = w.count;
            gw.C = a->dW + c0 * H; gw.ldc = H; gw.beta = 1;
            if ((e = launch_gemm<EPI_ACC>(gw, st)) != hipSuccess) return dev_fail(e, "dW");
        }
    }
    if (defer) {
        // the window's next chunk starts after this one's valid tokens
        hipLaunchKernelGGL(dw_fill_kernel, dim3(1), dim3(64), 0, st, wl.fill, w.count);
        if ((e = hipGetLastError()) != hipSuccess) return dev_fail(e, "dW window");
        // the host bound moves with the counter (the counter never passes it)
        win->reserved += reserve;
    }
    hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((H + 1023) / 1024), (unsigned)(n < 65535 ? n : 65535)),
                       dim3(256), 0, st, a->dh, H, w.dh_part, nsplit, n * H, w.inv, n, H, w.count, rule,
                       (int)al16(a->dh));
    if ((e = hipGetLastError()) != hipSuccess) return dev_fail(e, "dh splits");
    return ok();
}

}  // namespace
