// inkattn.hip -- learned-relative grouped-query attention forward with
// per-query sinks, for AMD CDNA4 (gfx950 / MI355X).
//
// Operation: forward of Inkling2FlexAttention (page
// "nemo_automodel.components.models.inkling2.flex_attention", section API),
// with the zero-valued virtual sink of Inkling2Attention.forward (page
// "nemo_automodel.components.models.inkling2.attention", v0.4) and the window
// of the sliding-window mask mod (page
// "nemo_automodel.components.attention.flex_attention").  The exact contract
// is in include/inkattn.h.
//
// Structure of one call:
//   1. summarize_kernel (scheduler pre-pass): per 32-token query block and per
//      64-key tile, the min / max document start column over real tokens and
//      the number of real tokens.  Every skip / full / masked decision of the
//      main kernel is taken from these summaries.
//   2. attn_fwd_kernel: one workgroup per (batch row, K/V head, head chunk,
//      32-token query block), one wave per query head of the chunk.  Each
//      64-key K/V tile is staged once in LDS and serves every query head of
//      the group (GQA).  Per wave and tile:
//        S^T = K Q^T      bf16 MFMA 32x32x16 (keys on M, queries on N), so that
//                         each lane owns one query column and row reductions
//                         are in-lane plus one exchange between wave halves;
//        + relative bias  gathered from the query's own profile row: for a
//                         32-key sub-tile the distances form one contiguous
//                         run per row;
//        mask             only on tiles classed as masked;
//        online softmax   running max / denominator per lane, started from
//                         the sink logit (the sink's weight enters the
//                         denominator, never the value sum);
//        O^T += V^T P^T   fp16 MFMA 32x32x16; P^T comes straight from the S^T
//                         accumulator registers (the key order inside each
//                         16-key step is permuted consistently on both
//                         operands), V is stored transposed in LDS.
//      Epilogue: out = O / l, lse = m + ln l.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdarg>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "inkattn.h"

namespace {

constexpr int BM = 32;   // query tokens per wave (MFMA N)
constexpr int BN = 64;   // keys per K/V tile (two MFMA M-blocks of 32)
constexpr int MAX_HPW = 8;  // query heads (waves) per workgroup, at most
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4_u __attribute__((ext_vector_type(4), aligned(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Per-tile summary written by the pre-pass: document start columns of the
// tile's real tokens (min, max) and how many real tokens it has.
struct __attribute__((aligned(16))) TileSummary {
    int amin, amax, nvalid, pad;
};

// ---------------------------------------------------------------------------
// Mask predicate shared by the attention kernel and the debug exports.
//
// gi_eff: global column of the query, or -1 for a query that is not real
//         (then no key passes the causal test).
// a_q:    the query's document start column gi - positions[i].
// j:      key column; c_k: the key's start column j - key_positions[j], or
//         INT_MIN for a key that is not real or lies past Sk.
// wlim:   window as an unsigned limit on gi - j (2^31 when there is none).
// Same document implies positions[i] - key_positions[j] == gi - j, so the
// window and causal tests both act on gi - j.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool key_visible(int gi_eff, int a_q, int j, int c_k, unsigned wlim)
{
    return (unsigned)(gi_eff - j) < wlim && c_k == a_q;
}

// Tile classes.
enum : int { TILE_SKIP = 0, TILE_MASKED = 1, TILE_FULL = 2 };

// Class of (query block, key tile) from the two summaries and the column
// ranges.  qlo / qhi: global columns of the block's first / last existing
// query; j0: first key column of the tile; key_hi: last existing key column.
__device__ __forceinline__ int classify_tile(const TileSummary& qs, int qlo, int qhi, int qcount,
                                             const TileSummary& ks, int j0, int key_hi, int kcount,
                                             int window)
{
    if (qs.nvalid == 0 || ks.nvalid == 0) return TILE_SKIP;
    if (j0 > qhi) return TILE_SKIP;                              // causal
    if (ks.amax < qs.amin || ks.amin > qs.amax) return TILE_SKIP;  // no common document
    if (window > 0 && qlo - key_hi >= window) return TILE_SKIP;  // nearest pair outside the window
    const bool one_doc = qs.amin == qs.amax && ks.amin == ks.amax && qs.amin == ks.amin;
    const bool all_real = qs.nvalid == qcount && ks.nvalid == kcount && qcount == BM && kcount == BN;
    const bool causal_full = key_hi <= qlo;
    const bool window_full = window <= 0 || qhi - j0 < window;
    return (one_doc && all_real && causal_full && window_full) ? TILE_FULL : TILE_MASKED;
}

// ---------------------------------------------------------------------------
// Scheduler pre-pass: one thread per (batch row, tile).
// ---------------------------------------------------------------------------
__global__ void summarize_kernel(const uint8_t* __restrict__ valid,
                                 const int32_t* __restrict__ positions,  // may be NULL: column
                                 int col0, int S, int B, int tile, int ntiles,
                                 TileSummary* __restrict__ out)
{
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= B * ntiles) return;
    const int b = idx / ntiles, t = idx - b * ntiles;
    int amin = INT_MAX, amax = INT_MIN, n = 0;
    const int lo = t * tile, hi = min(S, lo + tile);
    for (int i = lo; i < hi; ++i) {
        const size_t o = (size_t)b * S + i;
        if (!valid[o]) continue;
        const int col = col0 + i;
        const int a = positions ? col - positions[o] : 0;
        amin = min(amin, a);
        amax = max(amax, a);
        ++n;
    }
    TileSummary s;
    s.amin = amin; s.amax = amax; s.nvalid = n; s.pad = 0;
    out[idx] = s;
}

struct FwdParams {
    const __bf16* q;
    const __bf16* k;
    const __bf16* v;
    const void* profiles;
    const float* sink;
    const uint8_t* valid;
    const uint8_t* key_valid;
    const int32_t* positions;      // NULL: global column
    const int32_t* key_positions;  // NULL: key column
    const TileSummary* qsum;       // [B, nQB]
    const TileSummary* ksum;       // [B, nKT]
    float* out;
    float* lse;
    int B, Sq, Sk, Hq, Hkv, G, E;
    int window;      // <= 0: none
    int qoff;        // query_offset
    int hpw;         // query heads per workgroup (= waves)
    int nchunk;      // head chunks per K/V head (G / hpw)
    int nQB, nKT;
    float c_log2;    // head_dim^-0.5 * log2(e)
};

__device__ __forceinline__ float wave_half_swap(float x)
{
    return __shfl_xor(x, 32, 64);
}

template <int D, bool PROF_BF16>
__global__ __launch_bounds__(64 * MAX_HPW) void attn_fwd_kernel(FwdParams p)
{
    constexpr int NKK = D / 16;   // k-steps of S^T = K Q^T
    constexpr int NDB = D / 32;   // 32-row d-blocks of O^T
    constexpr int KS = D + 8;     // K row stride in LDS (bf16 elements)
    constexpr int VTS = BN + 4;   // V^T row stride in LDS (f16 elements)

    __shared__ __attribute__((aligned(16))) __bf16 k_lds[BN * KS];
    __shared__ __attribute__((aligned(16))) _Float16 vt_lds[D * VTS];
    __shared__ __attribute__((aligned(16))) int ca_lds[BN];

    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int qi = lane & 31;      // this lane's query within the block
    const int hh = lane >> 5;      // wave half

    // ---- work item: heads fastest so that consecutive workgroups share K/V
    // in one XCD's L2; query blocks in decreasing order (longest first).
    int idx = blockIdx.x;
    const int ngroups = p.Hkv * p.nchunk;
    const int hgi = idx % ngroups; idx /= ngroups;
    const int b = idx % p.B; idx /= p.B;
    const int qb = p.nQB - 1 - idx;
    const int g = hgi / p.nchunk;
    const int h = g * p.G + (hgi - g * p.nchunk) * p.hpw + wave;
    const int i0 = qb * BM;

    const int i = i0 + qi;
    const bool qin = i < p.Sq;
    const size_t qrow = (size_t)b * p.Sq + i;
    const int gi = p.qoff + i;
    const bool qreal = qin && p.valid[qrow] != 0;
    const int a_q = qreal ? (p.positions ? gi - p.positions[qrow] : 0) : 0;
    const int gi_eff = qreal ? gi : -1;
    const unsigned wlim = p.window > 0 ? (unsigned)p.window : 0x80000000u;
    const float sig = qin ? p.sink[qrow * p.Hq + h] : -INFINITY;

    // Q^T operand: lane holds q[i, h, 16*kk + 8*hh + 0..7].
    bf16x8 qreg[NKK];
    {
        const __bf16* qp = p.q + (qrow * p.Hq + h) * D + 8 * hh;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            if (qin) qreg[kk] = *(const bf16x8*)(qp + 16 * kk);
            else qreg[kk] = bf16x8{};
        }
    }

    // Online-softmax state (log2 units).  The sink's weight e^{s - m} counts
    // once, in the lower half's partial denominator.
    float m = sig * LOG2E;              // -inf when there is no sink
    float l = (hh == 0 && sig != -INFINITY) ? 1.0f : 0.0f;
    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};

    // ---- key-tile range of this query block
    const TileSummary qs = p.qsum[(size_t)b * p.nQB + qb];
    const int qcount = min(BM, p.Sq - i0);
    const int qlo = p.qoff + i0, qhi = p.qoff + i0 + qcount - 1;
    int jlo = 0;
    if (qs.nvalid > 0) jlo = max(jlo, qs.amin);            // key j >= its start column
    if (p.window > 0) jlo = max(jlo, qlo - p.window + 1);
    const int jhi = min(p.Sk - 1, qhi);
    const int kt_lo = jlo / BN;
    const int kt_hi = (qs.nvalid > 0 && jhi >= 0) ? jhi / BN : -1;

    const size_t prof_row = ((size_t)b * p.Hq + h) * p.Sq + i;  // row of profiles[b,h,i,:]

    for (int kt = kt_lo; kt <= kt_hi; ++kt) {
        const int j0 = kt * BN;
        const int kcount = min(BN, p.Sk - j0);
        const TileSummary ks = p.ksum[(size_t)b * p.nKT + kt];
        const int cls = classify_tile(qs, qlo, qhi, qcount, ks, j0, j0 + kcount - 1, kcount, p.window);
        if (cls == TILE_SKIP) continue;   // uniform over the workgroup

        // ---- stage K (row-major, padded) and V^T (fp16) for this tile
        __syncthreads();
        {
            constexpr int CPR = D / 8;   // 16-byte chunks per K row
            for (int c = tid; c < BN * CPR; c += nthr) {
                const int row = c / CPR, col = c - row * CPR;
                const int j = j0 + row;
                bf16x8 val = bf16x8{};
                if (row < kcount)
                    val = *(const bf16x8*)(p.k + (((size_t)b * p.Sk + j) * p.Hkv + g) * D + 8 * col);
                *(bf16x8*)(k_lds + row * KS + 8 * col) = val;
            }
            for (int u = tid; u < (BN / 4) * (D / 8); u += nthr) {
                const int kg = u & 15, dg = u >> 4;
                bf16x8 rows[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int jl = 4 * kg + rr;
                    const int j = j0 + jl;
                    bool ok = jl < kcount;
                    if (ok && cls != TILE_FULL) ok = p.key_valid[(size_t)b * p.Sk + j] != 0;
                    rows[rr] = ok ? *(const bf16x8*)(p.v + (((size_t)b * p.Sk + j) * p.Hkv + g) * D + 8 * dg)
                                  : bf16x8{};
                }
#pragma unroll
                for (int dd = 0; dd < 8; ++dd) {
                    f16x4 col;
                    col[0] = (_Float16)(float)rows[0][dd];
                    col[1] = (_Float16)(float)rows[1][dd];
                    col[2] = (_Float16)(float)rows[2][dd];
                    col[3] = (_Float16)(float)rows[3][dd];
                    *(f16x4*)(vt_lds + (8 * dg + dd) * VTS + 4 * kg) = col;
                }
            }
            if (cls == TILE_MASKED) {
                for (int t = tid; t < BN; t += nthr) {
                    const int j = j0 + t;
                    int c = INT_MIN;
                    if (t < kcount) {
                        const size_t o = (size_t)b * p.Sk + j;
                        if (p.key_valid[o]) c = p.key_positions ? j - p.key_positions[o] : 0;
                    }
                    ca_lds[t] = c;
                }
            }
        }
        __syncthreads();

        // ---- S^T = K Q^T for the two 32-key sub-tiles
        f32x16 sacc[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            sacc[s] = f32x16{};
            const __bf16* kp = k_lds + (32 * s + qi) * KS + 8 * hh;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const bf16x8 a = *(const bf16x8*)(kp + 16 * kk);
                sacc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kk], sacc[s], 0, 0, 0);
            }
        }

        // ---- logits in log2 units: u = (scale * s + bias) * log2(e)
        // Element (s, jj, e) is key j0 + 32 s + 8 jj + 4 hh + e.
        float u[2][16];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int js = j0 + 32 * s;
            const int rmin = qlo - (js + 31), rmax = qhi - js;   // distance range of the sub-tile
            const int R = gi - js;                               // this lane's distance to key js
            float bias[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) bias[t] = 0.0f;
            if (rmin < p.E) {
                if (rmin >= 0 && rmax < p.E) {
                    // every distance of the sub-tile lies inside [0, E): one run per 4 keys
                    if (qin) {
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            const int rb = R - 8 * jj - 4 * hh - 3;
                            if (PROF_BF16) {
                                const __bf16* pr = (const __bf16*)p.profiles + prof_row * p.E + rb;
#pragma unroll
                                for (int e = 0; e < 4; ++e) bias[4 * jj + e] = (float)pr[3 - e];
                            } else {
                                const f32x4_u w = *(const f32x4_u*)((const float*)p.profiles + prof_row * p.E + rb);
#pragma unroll
                                for (int e = 0; e < 4; ++e) bias[4 * jj + e] = w[3 - e];
                            }
                        }
                    }
                } else if (qin) {
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int r = R - 8 * jj - 4 * hh - e;
                            if (r >= 0 && r < p.E) {
                                if (PROF_BF16)
                                    bias[4 * jj + e] = (float)((const __bf16*)p.profiles)[prof_row * p.E + r];
                                else
                                    bias[4 * jj + e] = ((const float*)p.profiles)[prof_row * p.E + r];
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) u[s][t] = sacc[s][t] * p.c_log2 + bias[t] * LOG2E;
        }

        if (cls == TILE_MASKED) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int kl = 32 * s + 8 * jj + 4 * hh;
                    const i32x4 c4 = *(const i32x4*)(ca_lds + kl);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (!key_visible(gi_eff, a_q, j0 + kl + e, c4[e], wlim)) u[s][4 * jj + e] = -INFINITY;
                    }
                }
            }
        }

        // ---- online softmax (sink-initialised)
        float mx = -INFINITY;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int t = 0; t < 16; ++t) mx = fmaxf(mx, u[s][t]);
        mx = fmaxf(mx, wave_half_swap(mx));
        const float m_new = fmaxf(m, mx);
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m - m_use);
        float lsum = 0.0f;
        f16x8 pb[2][2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const float pv = __builtin_amdgcn_exp2f(u[s][t] - m_use);
                lsum += pv;
                // 16-key step c of sub-tile s takes elements jj = 2c, 2c+1
                pb[s][t >> 3][t & 7] = (_Float16)pv;
            }
        }
        l = l * alpha + lsum;
        if (__builtin_amdgcn_ballot_w64(m_new > m) != 0) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int t = 0; t < 16; ++t) oacc[db][t] *= alpha;
        }
        m = m_new;

        // ---- O^T += V^T P^T
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int kb = 32 * s + 16 * c + 4 * hh;
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const _Float16* vp = vt_lds + (32 * db + qi) * VTS + kb;
                    const f16x4 lo = *(const f16x4*)(vp);
                    const f16x4 hi = *(const f16x4*)(vp + 8);
                    const f16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[s][c], oacc[db], 0, 0, 0);
                }
            }
        }
    }

    // ---- epilogue
    const float l_tot = l + wave_half_swap(l);
    if (!qin) return;
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    float* op = p.out + (qrow * p.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            f32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = oacc[db][4 * jj + e] * inv;
            *(f32x4*)(op + 32 * db + 8 * jj + 4 * hh) = w;
        }
    }
    if (hh == 0) {
        float lse;
        if (!qreal) lse = sig;
        else if (l_tot > 0.0f) lse = (m + log2f(l_tot)) * LN2;
        else lse = -INFINITY;
        p.lse[qrow * p.Hq + h] = lse;
    }
}

// ---------------------------------------------------------------------------
// Debug exports
// ---------------------------------------------------------------------------
__global__ void debug_counts_kernel(const uint8_t* __restrict__ valid, const uint8_t* __restrict__ key_valid,
                                    const int32_t* __restrict__ positions, const int32_t* __restrict__ key_positions,
                                    int window, int qoff, int B, int Sq, int Sk, int32_t* __restrict__ n_allowed)
{
    const int row = blockIdx.x;     // b * Sq + i
    const int b = row / Sq, i = row - b * Sq;
    const size_t qrow = (size_t)b * Sq + i;
    const int gi = qoff + i;
    const bool qreal = valid[qrow] != 0;
    const int a_q = qreal ? (positions ? gi - positions[qrow] : 0) : 0;
    const int gi_eff = qreal ? gi : -1;
    const unsigned wlim = window > 0 ? (unsigned)window : 0x80000000u;
    int cnt = 0;
    for (int j = threadIdx.x; j < Sk; j += blockDim.x) {
        const size_t o = (size_t)b * Sk + j;
        const int c = key_valid[o] ? (key_positions ? j - key_positions[o] : 0) : INT_MIN;
        cnt += key_visible(gi_eff, a_q, j, c, wlim) ? 1 : 0;
    }
    __shared__ int red[256];
    red[threadIdx.x] = cnt;
    __syncthreads();
    for (int w = blockDim.x / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) n_allowed[qrow] = red[0];
}

__global__ void debug_tiles_kernel(const TileSummary* __restrict__ qsum, const TileSummary* __restrict__ ksum,
                                   int window, int qoff, int B, int Sq, int Sk, int nQB, int nKT,
                                   uint8_t* __restrict__ tile_class)
{
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)B * nQB * nKT) return;
    const int kt = (int)(idx % nKT);
    const int qb = (int)((idx / nKT) % nQB);
    const int b = (int)(idx / ((size_t)nKT * nQB));
    const TileSummary qs = qsum[(size_t)b * nQB + qb];
    const TileSummary ks = ksum[(size_t)b * nKT + kt];
    const int i0 = qb * BM;
    const int qcount = min(BM, Sq - i0);
    const int j0 = kt * BN;
    const int kcount = min(BN, Sk - j0);
    tile_class[idx] = (uint8_t)classify_tile(qs, qoff + i0, qoff + i0 + qcount - 1, qcount, ks, j0,
                                             j0 + kcount - 1, kcount, window);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

size_t summaries_bytes(int B, int Sq, int Sk)
{
    const size_t nq = (size_t)B * ceil_div(Sq, BM);
    const size_t nk = (size_t)B * ceil_div(Sk, BN);
    return (nq + nk) * sizeof(TileSummary);
}

// Defaults of the optional arguments and the checks shared by every entry point.
struct MaskArgs {
    const uint8_t* key_valid;
    const int32_t* positions;
    const int32_t* key_positions;
};

int resolve_mask_args(const uint8_t* valid, const uint8_t* key_valid, const int32_t* positions,
                      const int32_t* key_positions, int64_t window, int64_t query_offset,
                      int B, int Sq, int Sk, MaskArgs* outa)
{
    if (B < 0 || Sq < 0 || Sk < 0) return fail(INKATTN_ERR_SHAPE, "negative size (B=%d Sq=%d Sk=%d)", B, Sq, Sk);
    if (Sq >= (1 << 30) || Sk >= (1 << 30)) return fail(INKATTN_ERR_SHAPE, "Sq / Sk must be below 2^30");
    if (query_offset < 0 || query_offset + Sq >= (int64_t(1) << 30))
        return fail(INKATTN_ERR_SHAPE, "query_offset must be >= 0 and query_offset + Sq below 2^30");
    if ((size_t)B * Sq > 0 && !valid) return fail(INKATTN_ERR_NULL, "valid is NULL");
    const bool same_tokens = (Sk == Sq && query_offset == 0);
    MaskArgs a;
    a.key_valid = key_valid;
    a.positions = positions;
    a.key_positions = key_positions;
    if (!key_valid && Sk > 0) {
        if (!same_tokens)
            return fail(INKATTN_ERR_NULL, "key_valid must be given when Sk != Sq or query_offset != 0");
        a.key_valid = valid;
    }
    if (!key_positions && same_tokens) a.key_positions = positions;
    if (positions && !aligned(positions, 4)) return fail(INKATTN_ERR_ALIGN, "positions not 4-byte aligned");
    if (a.key_positions && !aligned(a.key_positions, 4))
        return fail(INKATTN_ERR_ALIGN, "key_positions not 4-byte aligned");
    *outa = a;
    return INKATTN_OK;
}

int check_launch(const char* what)
{
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(INKATTN_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    return INKATTN_OK;
}

int launch_summaries(const uint8_t* valid, const int32_t* positions, const uint8_t* key_valid,
                     const int32_t* key_positions, int qoff, int B, int Sq, int Sk,
                     TileSummary* qsum, TileSummary* ksum, hipStream_t st)
{
    const int nQB = ceil_div(Sq, BM), nKT = ceil_div(Sk, BN);
    if (B * nQB > 0) {
        const int n = B * nQB;
        hipLaunchKernelGGL(summarize_kernel, dim3(ceil_div(n, 256)), dim3(256), 0, st,
                           valid, positions, qoff, Sq, B, BM, nQB, qsum);
        if (int rc = check_launch("summarize_kernel(queries)")) return rc;
    }
    if (B * nKT > 0) {
        const int n = B * nKT;
        hipLaunchKernelGGL(summarize_kernel, dim3(ceil_div(n, 256)), dim3(256), 0, st,
                           key_valid, key_positions, 0, Sk, B, BN, nKT, ksum);
        if (int rc = check_launch("summarize_kernel(keys)")) return rc;
    }
    return INKATTN_OK;
}

int heads_per_workgroup(int G)
{
    for (int d = MAX_HPW; d >= 1; --d)
        if (G % d == 0) return d;
    return 1;
}

}  // namespace

extern "C" {

size_t attn_fwd_workspace_size(int B, int Sq, int Sk)
{
    if (B <= 0 || Sq < 0 || Sk < 0) return 0;
    return summaries_bytes(B, Sq, Sk);
}

int attn_query_block(void) { return BM; }
int attn_key_tile(void) { return BN; }

const char* attn_status_string(int status)
{
    switch (status) {
    case INKATTN_OK: return "ok";
    case INKATTN_ERR_NULL: return "required pointer is NULL";
    case INKATTN_ERR_SHAPE: return "inconsistent or out-of-range sizes";
    case INKATTN_ERR_UNSUPPORTED: return "unsupported head_dim or dtype";
    case INKATTN_ERR_ALIGN: return "pointer misaligned";
    case INKATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case INKATTN_ERR_LAUNCH: return "HIP launch failed";
    default: return "unknown status";
    }
}

const char* attn_last_error(void) { return g_last_error; }

int attn_plan(const uint8_t* valid, const uint8_t* key_valid,
              const int32_t* positions, const int32_t* key_positions,
              int64_t query_offset, int B, int Sq, int Sk,
              void* workspace, size_t workspace_bytes, void* stream)
{
    g_last_error[0] = '\0';
    MaskArgs ma;
    if (int rc = resolve_mask_args(valid, key_valid, positions, key_positions, 0, query_offset, B, Sq, Sk, &ma))
        return rc;
    if ((size_t)B * (Sq + Sk) == 0) return INKATTN_OK;
    const size_t need = summaries_bytes(B, Sq, Sk);
    if (!workspace || workspace_bytes < need)
        return fail(INKATTN_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
    if (!aligned(workspace, 16)) return fail(INKATTN_ERR_ALIGN, "workspace not 16-byte aligned");
    const int nQB = ceil_div(Sq, BM);
    TileSummary* qsum = (TileSummary*)workspace;
    TileSummary* ksum = qsum + (size_t)B * nQB;
    return launch_summaries(valid, positions, ma.key_valid, ma.key_positions, (int)query_offset, B, Sq, Sk,
                            qsum, ksum, (hipStream_t)stream);
}

int attn_fwd_planned(const void* q, const void* k, const void* v,
                     const void* profiles, int profiles_dtype,
                     const float* sink, const uint8_t* valid, const uint8_t* key_valid,
                     const int32_t* positions, const int32_t* key_positions,
                     int64_t window, int64_t query_offset,
                     int B, int Sq, int Sk, int Hq, int Hkv, int D, int E,
                     float* out, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream)
{
    g_last_error[0] = '\0';
    if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
        return fail(INKATTN_ERR_SHAPE, "Hq=%d must be a positive multiple of Hkv=%d", Hq, Hkv);
    if (E < 1) return fail(INKATTN_ERR_SHAPE, "relative extent E=%d must be >= 1", E);
    if (D != 64 && D != 128) return fail(INKATTN_ERR_UNSUPPORTED, "head_dim %d not built (64, 128)", D);
    if (profiles_dtype != INKATTN_F32 && profiles_dtype != INKATTN_BF16)
        return fail(INKATTN_ERR_UNSUPPORTED, "profiles dtype %d unknown", profiles_dtype);
    MaskArgs ma;
    if (int rc = resolve_mask_args(valid, key_valid, positions, key_positions, window, query_offset,
                                   B, Sq, Sk, &ma))
        return rc;
    if (window >= (int64_t(1) << 31) || window < 0) window = 0;
    const size_t nq_elems = (size_t)B * Sq * Hq * D;
    const size_t np_elems = (size_t)B * Hq * Sq * E;
    if (nq_elems >= (size_t(1) << 40) || np_elems >= (size_t(1) << 40))
        return fail(INKATTN_ERR_SHAPE, "tensor too large");
    if ((size_t)B * Sq == 0) return INKATTN_OK;   // nothing to write
    if (!q || !profiles || !sink || !out || !lse) return fail(INKATTN_ERR_NULL, "q/profiles/sink/out/lse is NULL");
    if (Sk > 0 && (!k || !v)) return fail(INKATTN_ERR_NULL, "k or v is NULL");
    if (!aligned(q, 16) || (Sk > 0 && (!aligned(k, 16) || !aligned(v, 16))) || !aligned(out, 16))
        return fail(INKATTN_ERR_ALIGN, "q, k, v and out must be 16-byte aligned");
    if (!aligned(profiles, profiles_dtype == INKATTN_F32 ? 4 : 2) || !aligned(sink, 4) || !aligned(lse, 4))
        return fail(INKATTN_ERR_ALIGN, "profiles / sink / lse misaligned");
    const size_t need = summaries_bytes(B, Sq, Sk);
    if (!workspace || workspace_bytes < need)
        return fail(INKATTN_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
    if (!aligned(workspace, 16)) return fail(INKATTN_ERR_ALIGN, "workspace not 16-byte aligned");

    hipStream_t st = (hipStream_t)stream;
    const int nQB = ceil_div(Sq, BM), nKT = ceil_div(Sk, BN);
    TileSummary* qsum = (TileSummary*)workspace;
    TileSummary* ksum = qsum + (size_t)B * nQB;

    FwdParams p;
    p.q = (const __bf16*)q;
    p.k = (const __bf16*)k;
    p.v = (const __bf16*)v;
    p.profiles = profiles;
    p.sink = sink;
    p.valid = valid;
    p.key_valid = ma.key_valid;
    p.positions = positions;
    p.key_positions = ma.key_positions;
    p.qsum = qsum;
    p.ksum = ksum;
    p.out = out;
    p.lse = lse;
    p.B = B; p.Sq = Sq; p.Sk = Sk; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv; p.E = E;
    p.window = (int)window;
    p.qoff = (int)query_offset;
    p.hpw = heads_per_workgroup(p.G);
    p.nchunk = p.G / p.hpw;
    p.nQB = nQB; p.nKT = nKT;
    p.c_log2 = (float)(1.0 / std::sqrt((double)D) * 1.4426950408889634);

    const size_t nblocks = (size_t)nQB * B * Hkv * p.nchunk;
    if (nblocks >= (size_t(1) << 31)) return fail(INKATTN_ERR_SHAPE, "grid too large");
    const dim3 grid((unsigned)nblocks), block(64 * p.hpw);
    const bool pb = profiles_dtype == INKATTN_BF16;
    if (D == 128) {
        if (pb) hipLaunchKernelGGL((attn_fwd_kernel<128, true>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((attn_fwd_kernel<128, false>), grid, block, 0, st, p);
    } else {
        if (pb) hipLaunchKernelGGL((attn_fwd_kernel<64, true>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((attn_fwd_kernel<64, false>), grid, block, 0, st, p);
    }
    return check_launch("attn_fwd_kernel");
}

int attn_fwd(const void* q, const void* k, const void* v,
             const void* profiles, int profiles_dtype,
             const float* sink, const uint8_t* valid, const uint8_t* key_valid,
             const int32_t* positions, const int32_t* key_positions,
             int64_t window, int64_t query_offset,
             int B, int Sq, int Sk, int Hq, int Hkv, int D, int E,
             float* out, float* lse,
             void* workspace, size_t workspace_bytes, void* stream)
{
    // Validate everything before enqueuing the pre-pass: a rejected call enqueues nothing.
    g_last_error[0] = '\0';
    if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
        return fail(INKATTN_ERR_SHAPE, "Hq=%d must be a positive multiple of Hkv=%d", Hq, Hkv);
    if (E < 1) return fail(INKATTN_ERR_SHAPE, "relative extent E=%d must be >= 1", E);
    if (D != 64 && D != 128) return fail(INKATTN_ERR_UNSUPPORTED, "head_dim %d not built (64, 128)", D);
    if (profiles_dtype != INKATTN_F32 && profiles_dtype != INKATTN_BF16)
        return fail(INKATTN_ERR_UNSUPPORTED, "profiles dtype %d unknown", profiles_dtype);
    MaskArgs ma;
    if (int rc = resolve_mask_args(valid, key_valid, positions, key_positions, window, query_offset,
                                   B, Sq, Sk, &ma))
        return rc;
    if ((size_t)B * Sq == 0) return INKATTN_OK;
    if (!q || !profiles || !sink || !out || !lse) return fail(INKATTN_ERR_NULL, "q/profiles/sink/out/lse is NULL");
    if (Sk > 0 && (!k || !v)) return fail(INKATTN_ERR_NULL, "k or v is NULL");
    if (!aligned(q, 16) || (Sk > 0 && (!aligned(k, 16) || !aligned(v, 16))) || !aligned(out, 16))
        return fail(INKATTN_ERR_ALIGN, "q, k, v and out must be 16-byte aligned");
    if (!aligned(profiles, profiles_dtype == INKATTN_F32 ? 4 : 2) || !aligned(sink, 4) || !aligned(lse, 4))
        return fail(INKATTN_ERR_ALIGN, "profiles / sink / lse misaligned");
    const size_t need = summaries_bytes(B, Sq, Sk);
    if (!workspace || workspace_bytes < need)
        return fail(INKATTN_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
    if (!aligned(workspace, 16)) return fail(INKATTN_ERR_ALIGN, "workspace not 16-byte aligned");
    if (int rc = attn_plan(valid, key_valid, positions, key_positions, query_offset, B, Sq, Sk, workspace,
                           workspace_bytes, stream))
        return rc;
    return attn_fwd_planned(q, k, v, profiles, profiles_dtype, sink, valid, key_valid, positions, key_positions,
                            window, query_offset, B, Sq, Sk, Hq, Hkv, D, E, out, lse, workspace, workspace_bytes,
                            stream);
}

int attn_debug_counts(const uint8_t* valid, const uint8_t* key_valid,
                      const int32_t* positions, const int32_t* key_positions,
                      int64_t window, int64_t query_offset, int B, int Sq, int Sk,
                      int32_t* n_allowed, void* stream)
{
    g_last_error[0] = '\0';
    MaskArgs ma;
    if (int rc = resolve_mask_args(valid, key_valid, positions, key_positions, window, query_offset,
                                   B, Sq, Sk, &ma))
        return rc;
    if (window >= (int64_t(1) << 31) || window < 0) window = 0;
    if ((size_t)B * Sq == 0) return INKATTN_OK;
    if (!n_allowed) return fail(INKATTN_ERR_NULL, "n_allowed is NULL");
    if (!aligned(n_allowed, 4)) return fail(INKATTN_ERR_ALIGN, "n_allowed not 4-byte aligned");
    if ((size_t)B * Sq >= (size_t(1) << 31)) return fail(INKATTN_ERR_SHAPE, "too many rows");
    hipLaunchKernelGGL(debug_counts_kernel, dim3(B * Sq), dim3(256), 0, (hipStream_t)stream, valid,
                       ma.key_valid, positions, ma.key_positions, (int)window, (int)query_offset, B, Sq, Sk,
                       n_allowed);
    return check_launch("debug_counts_kernel");
}

int attn_debug_tiles(const uint8_t* valid, const uint8_t* key_valid,
                     const int32_t* positions, const int32_t* key_positions,
                     int64_t window, int64_t query_offset, int B, int Sq, int Sk,
                     uint8_t* tile_class, void* workspace, size_t workspace_bytes,
                     void* stream)
{
    g_last_error[0] = '\0';
    MaskArgs ma;
    if (int rc = resolve_mask_args(valid, key_valid, positions, key_positions, window, query_offset,
                                   B, Sq, Sk, &ma))
        return rc;
    if (window >= (int64_t(1) << 31) || window < 0) window = 0;
    const int nQB = ceil_div(Sq, BM), nKT = ceil_div(Sk, BN);
    const size_t n = (size_t)B * nQB * nKT;
    if (n == 0) return INKATTN_OK;
    if (!tile_class) return fail(INKATTN_ERR_NULL, "tile_class is NULL");
    const size_t need = summaries_bytes(B, Sq, Sk);
    if (!workspace || workspace_bytes < need)
        return fail(INKATTN_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
    if (!aligned(workspace, 16)) return fail(INKATTN_ERR_ALIGN, "workspace not 16-byte aligned");
    if (n >= (size_t(1) << 40)) return fail(INKATTN_ERR_SHAPE, "too many tiles");
    hipStream_t st = (hipStream_t)stream;
    TileSummary* qsum = (TileSummary*)workspace;
    TileSummary* ksum = qsum + (size_t)B * nQB;
    if (int rc = launch_summaries(valid, positions, ma.key_valid, ma.key_positions, (int)query_offset,
                                  B, Sq, Sk, qsum, ksum, st))
        return rc;
    hipLaunchKernelGGL(debug_tiles_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, qsum, ksum,
                       (int)window, (int)query_offset, B, Sq, Sk, nQB, nKT, tile_class);
    return check_launch("debug_tiles_kernel");
}

}  // extern "C"
