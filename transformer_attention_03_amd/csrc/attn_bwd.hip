// attn_bwd.hip -- gradients of the learned-relative grouped-query attention
// with per-query sinks, for AMD CDNA4 (gfx950 / MI355X).
//
// Operation: the backward of the forward in inkattn.hip.  The page
// "nemo_automodel.components.models.inkling2.flex_attention" (module summary
// and class Inkling2FlexAttention) makes the per-query sinks differentiable
// and lets gradients reach the captured profiles and flow in through the
// returned log-sum-exp.  With z_ij = scale <q_i, k_j> + bias_ij the allowed
// logits, P_ij = e^{z_ij - lse_i} the weights of the forward (lse includes the
// sink sigma_i) and upstream gradients dout, dlse:
//   Delta_i  = <dout_i, out_i>
//   dz_ij    = P_ij (<dout_i, v_j> - Delta_i + dlse_i)
//   dq_i     = scale sum_j dz_ij k_j     dk_j = scale sum_i dz_ij q_i
//   dv_j     = sum_i P_ij dout_i
//   dprofiles[b,h,i,r] = dz_ij for the key j at distance r, 0 where none is
//   dsink_i  = e^{sigma_i - lse_i} (dlse_i - Delta_i)
//
// Structure of one call:
//   1. summarize_kernel (the forward's pre-pass): mask summaries per tile.
//   2. bwd_prep_kernel: per row Delta - dlse, dsink and lse * log2(e); dout
//      rounded to bf16 rows (0 on rows that are not real); per query its
//      global column (-1 if not real) and document start column.
//   3. bwd_dq_kernel (query-parallel, two waves per (query head, 32
//      queries), one per 32-key half of each tile, keys on MFMA M as in the
//      forward): per 64-key tile S^T = K Q^T and dP^T = V dO^T, then P and dS
//      from the saved lse, dS written to the profile gradient row (a
//      contiguous run per query), dQ^T += K^T dS^T with K^T read from the
//      staged K rows by transposing LDS reads; the halves' partials are
//      summed at the end.  Each wave's bias runs arrive by LDS DMA two tiles
//      ahead (two strips per wave).  Every entry of a query's profile-gradient row is
//      written by one of its two waves: zeros where no tile they visit puts
//      a value.
//   4. bwd_dkdv_kernel (key-parallel, two waves per 32 keys, queries on MFMA
//      M): per (32-query block, head of the group) the P wave forms S = Q K^T
//      and P and accumulates dV^T += dO^T P; the dS wave forms dP = dO V^T,
//      takes P through LDS one block later, forms dS and accumulates
//      dK^T += Q^T dS.  The transposed operands are read from the staged rows
//      with transposing LDS reads; the stages come by LDS DMA through a ring
//      of four, two ahead.
// Products are bf16 MFMA 32x32x16 with fp32 accumulation; P and dS are
// rounded to bf16 for the products that consume them.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>
#include <climits>
#include <cmath>
#include <cstdint>

#include "common.h"
#include "inkattn.h"

namespace {

using namespace inkattn;

constexpr int BW_WAVES = 4;          // (query head, 32-query block) units per dQ workgroup
constexpr int DQ_WAVES = 2 * BW_WAVES; // dQ waves: one per unit and 32-key half of each tile
// bias class of a tile for one wave: no distance inside [0, E), all inside, mixed
enum : int { BC_NONE = 0, BC_FULL = 1, BC_EDGE = 2 };
constexpr int KV_WAVES = 8;          // waves per dK / dV workgroup (two per 32-key group)
constexpr int KV_KEYS = 128;         // keys per dK / dV workgroup

struct BwdParams {
    const __bf16* q;               // [B, Sq, Hq, D]
    const __bf16* k;               // [B, Sk, Hkv, D]
    const __bf16* v;               // [B, Sk, Hkv, D]
    const void* profiles;          // [B, Hq, Sq, E] fp32 or bf16
    const float* sink;             // [B, Sq, Hq]
    const float* out;              // [B, Sq, Hq, D]
    const float* lse;              // [B, Sq, Hq]
    const float* dout;             // [B, Sq, Hq, D]
    const float* dlse;             // [B, Sq, Hq] or NULL
    const uint8_t* valid;          // [B, Sq]
    const uint8_t* key_valid;      // [B, Sk]
    const int32_t* positions;      // [B, Sq] or NULL (global column)
    const TileSummary* qsum;       // [B, nQB]
    const TileSummary* ksum;       // [B, nKT]
    const int* kanchor;            // [B, nKT * 64] key start column, INT_MIN if not real
    int2* qinfo;                   // [B, Sq] {global column or -1, document start column}
    float2* rowstat;               // [B, Hq, Sq] {lse * log2(e) (0 when lse = -inf), Delta - dlse}
    __bf16* dob;                   // [B, Sq, Hq, D] bf16 dout, 0 on rows that are not real
    float* dq;                     // [B, Sq, Hq, D]
    float* dk;                     // [B, Sk, Hkv, D]
    float* dv;                     // [B, Sk, Hkv, D]
    void* dprofiles;               // [B, Hq, Sq, E], dtype of profiles
    float* dsink;                  // [B, Sq, Hq]
    int B, Sq, Sk, Hq, Hkv, G, E;
    int window;                    // <= 0: none
    int qoff;
    int hpw, tpw, nchunk, nQG;     // dQ workgroup shape (as the forward's)
    int nQB, nKT, nKB;
    float scale;                   // head_dim^-0.5
    float c_log2;                  // scale * log2(e)
};

// XOR swizzle of the 16-byte chunks of a staged row of D bf16 (row pitch
// 2 D bytes).  D = 128: the two 2-bit fields of r mod 16 are swapped, so that
// 16 consecutive rows read at one logical chunk hit 16 distinct groups of 4
// banks, and so do 4 consecutive rows read at 4 consecutive logical chunks
// (the pattern of a transposing read).
// Slot permutation of the 16-byte chunks of a 128-byte whole-run row in a
// bias strip: 8 consecutive rows (from a multiple of 8) read at one chunk
// index hit 8 distinct slots, and 16 consecutive rows hit each slot once
// from an even and once from an odd row, so that neither a 128-byte nor a
// 256-byte bank period leaves two lanes of a group on the same banks.
__device__ __forceinline__ unsigned run_swz(unsigned r) { return (r & 7u) ^ ((r >> 3) & 1u); }

template <int D> __device__ __forceinline__ int row_swz(int r)
{
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((r >> 1) & 7);
}

// Transposing reads of staged rows (D = 128: pitch 256 bytes, chunks placed by
// row_swz): lane ln reads 8 bytes of row 16 c + 8 hi + 4 (ln / 32) +
// (ln % 16) / 4 at the columns 32 db + 16 ((ln / 16) % 2) + 4 (ln % 4).  With
// t = (ln / 4) % 4 and y = 2 ((ln / 16) % 2) + (ln / 2) % 2 the row's swizzle
// is 4 t + 2 hi + ln / 32 and the column chunk 4 db + y, so the byte offset is
// 4096 c + 2048 hi + 1024 (ln / 32) + 256 t + 64 (db ^ t) + 16 (y ^ (ln / 32)
// ^ 2 hi) + 8 (ln % 2) = (tr_base128(ln) + 2048 hi) ^ (64 db + 32 hi) + 4096 c:
// c, hi and db enter as constants (the XOR only touches bits 4..7, which the
// row terms and a row base that is a multiple of 256 leave clear).
__device__ __forceinline__ unsigned tr_base128(unsigned ln)
{
    const unsigned hh = ln >> 5, t = (ln >> 2) & 3u, y = 2u * ((ln >> 4) & 1u) + ((ln >> 1) & 1u);
    return 1024u * hh + 320u * t + 16u * (y ^ hh) + 8u * (ln & 1u);
}

// ---------------------------------------------------------------------------
// Row statistics, bf16 dout, query descriptors.  TPR = D / 4 threads per
// (batch row, query, head) row.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p)
{
    constexpr int TPR = D / 4;
    const long long row = (long long)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;   // (b Sq + i) Hq + h
    const int t = threadIdx.x % TPR;
    if (row >= (long long)p.B * p.Sq * p.Hq) return;   // a row's threads leave together
    const int h = (int)(row % p.Hq);
    const long long bi = row / p.Hq;
    const int i = (int)(bi % p.Sq);
    const int b = (int)(bi / p.Sq);
    const bool real = p.valid[bi] != 0;
    const f32x4 go = *(const f32x4*)(p.dout + row * D + 4 * t);
    const f32x4 o = *(const f32x4*)(p.out + row * D + 4 * t);
    float dot = go[0] * o[0] + go[1] * o[1] + go[2] * o[2] + go[3] * o[3];
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) dot += __shfl_xor(dot, off, TPR);
    if (!real) dot = 0.0f;   // a row that is not real has out = 0; its dout is ignored
    bf16x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = real ? (__bf16)go[e] : (__bf16)0.0f;   // round to nearest even
    *(bf16x4*)(p.dob + row * D + 4 * t) = w;
    if (t == 0) {
        const float L = p.lse[row];
        const float sg = p.sink[row];
        const float dl = p.dlse ? p.dlse[row] : 0.0f;
        const bool fin = L > -INFINITY;
        p.dsink[row] = fin ? expf(sg - L) * (dl - dot) : 0.0f;
        p.rowstat[((long long)b * p.Hq + h) * p.Sq + i] = make_float2(fin ? L * LOG2E : 0.0f, dot - dl);
        if (h == 0) {
            const int gi = p.qoff + i;
            p.qinfo[bi] = make_int2(real ? gi : -1, real ? (p.positions ? gi - p.positions[bi] : 0) : 0);
        }
    }
}

// Waits until at most n vector-memory instructions of the wave are
// outstanding (n in {0, 4, 8, 16, 20, 32}: the counts an iteration of the dQ
// kernel can leave in flight), then meets the workgroup.  s_waitcnt operand:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 (7: no wait), lgkmcnt 11:8 (0).
__device__ __forceinline__ void wait_vm_and_barrier(int n)
{
#if defined(__HIP_DEVICE_COMPILE__)
    switch (n) {
    case 4: __builtin_amdgcn_s_waitcnt(0x0074); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0078); break;
    case 16: __builtin_amdgcn_s_waitcnt(0x4070); break;
    case 20: __builtin_amdgcn_s_waitcnt(0x4074); break;
    case 32: __builtin_amdgcn_s_waitcnt(0x8070); break;
    default: __builtin_amdgcn_s_waitcnt(0x0070); break;
    }
#endif
    asm volatile("s_barrier" ::: "memory");
}

// Per-workgroup list of live tiles, built in rounds of NSCHED candidates (one
// per thread) between barriers.  An entry is (candidate - base) in bits 0..15
// and a 2-bit class per wave group in bits 16 + 2 x.
template <int NSCHED>
struct Schedule {
    int* list;     // NSCHED entries + one count per wave
    int base, n, i;
};

// Builds the round of candidates base .. base + NSCHED - 1 (classify returns
// the entry's class bits, 0 for a dead candidate, or -1 past the end).
template <int NSCHED, typename F>
__device__ __forceinline__ void build_round(Schedule<NSCHED>& s, F classify)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int code = classify(s.base + tid);
    const bool live = code > 0;
    const unsigned long long bal = __builtin_amdgcn_ballot_w64(live);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    __syncthreads();                                   // the previous round's entries are read
    if (lane == 0) s.list[NSCHED + wave] = __popcll(bal);
    __syncthreads();
    int off = 0, total = 0;
    for (int w = 0; w < NSCHED / 64; ++w) {
        const int cw = s.list[NSCHED + w];
        off += w < wave ? cw : 0;
        total += cw;
    }
    if (live) s.list[off + before] = (code << 16) | tid;
    __syncthreads();
    s.n = __builtin_amdgcn_readfirstlane(total);
    s.i = 0;
}

// Next live entry (candidate index and class bits), or {-1, 0} at the end.
template <int NSCHED, typename F>
__device__ __forceinline__ int2 next_entry(Schedule<NSCHED>& s, int last, F classify)
{
    while (s.i >= s.n && s.base <= last) {
        build_round(s, classify);
        s.base += NSCHED;
    }
    if (s.i < s.n) {
        const unsigned w = (unsigned)__builtin_amdgcn_readfirstlane(s.list[s.i]);
        ++s.i;
        return make_int2(s.base - NSCHED + (int)(w & 0xFFFFu), (int)(w >> 16));
    }
    return make_int2(-1, 0);
}

// Bias entry of a (query row, distance r) as float: 0 outside [0, E).
template <bool PB>
__device__ __forceinline__ float bias_at(const void* prow, int r, int E)
{
    if ((unsigned)r >= (unsigned)E) return 0.0f;
    if constexpr (PB) return (float)((const __bf16*)prow)[r];
    else return ((const float*)prow)[r];
}

template <bool PB>
__device__ __forceinline__ void store_grad(void* prow, int r, float x)
{
    if constexpr (PB) ((__bf16*)prow)[r] = (__bf16)x;
    else ((float*)prow)[r] = x;
}

// N (4 or 8) transposing LDS reads (ds_read_b64_tr_b16) at the LDS byte addresses
// a[], and the wait for them, in one asm block.  Through the builtin, the
// compiler puts a wait for every outstanding vector-memory instruction before
// each such read (it cannot tell the read from the LDS the DMA is still
// writing), which would hold the DMA sent ahead for later tiles; the reads
// here only touch data whose DMA has landed.  The outputs are written when the
// block ends (its own wait), and none overlaps an address (early clobber).
// OFF (a multiple of 8 below 65536) is added to every address by the
// instructions' offset field.
template <int N, int OFF = 0>
__device__ __forceinline__ void tr_read(s16x4 (&r)[N], const unsigned (&a)[N])
{
    static_assert(N == 4 || N == 8, "four or eight reads");
    static_assert(OFF >= 0 && OFF < 65536 && OFF % 8 == 0, "offset field");
#if defined(__HIP_DEVICE_COMPILE__)
    if constexpr (N == 4) {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %4 offset:%8\n\t"
            "ds_read_b64_tr_b16 %1, %5 offset:%8\n\t"
            "ds_read_b64_tr_b16 %2, %6 offset:%8\n\t"
            "ds_read_b64_tr_b16 %3, %7 offset:%8\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
            : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF)
            : "memory");
        return;
    } else
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%16\n\t"
        "ds_read_b64_tr_b16 %1, %9 offset:%16\n\t"
        "ds_read_b64_tr_b16 %2, %10 offset:%16\n\t"
        "ds_read_b64_tr_b16 %3, %11 offset:%16\n\t"
        "ds_read_b64_tr_b16 %4, %12 offset:%16\n\t"
        "ds_read_b64_tr_b16 %5, %13 offset:%16\n\t"
        "ds_read_b64_tr_b16 %6, %14 offset:%16\n\t"
        "ds_read_b64_tr_b16 %7, %15 offset:%16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "i"(OFF)
        : "memory");
#else
    for (int x = 0; x < N; ++x) r[x] = s16x4{};
    (void)a;
#endif
}

// The same for N (4 or 8) 16-byte LDS reads at the byte addresses a[].
template <int N>
__device__ __forceinline__ void lds_read16(bf16x8 (&r)[N], const unsigned (&a)[N])
{
    static_assert(N == 4 || N == 8, "four or eight reads");
#if defined(__HIP_DEVICE_COMPILE__)
    if constexpr (N == 4) {
        asm volatile(
            "ds_read_b128 %0, %4\n\t"
            "ds_read_b128 %1, %5\n\t"
            "ds_read_b128 %2, %6\n\t"
            "ds_read_b128 %3, %7\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
            : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
            : "memory");
    } else {
        asm volatile(
            "ds_read_b128 %0, %8\n\t"
            "ds_read_b128 %1, %9\n\t"
            "ds_read_b128 %2, %10\n\t"
            "ds_read_b128 %3, %11\n\t"
            "ds_read_b128 %4, %12\n\t"
            "ds_read_b128 %5, %13\n\t"
            "ds_read_b128 %6, %14\n\t"
            "ds_read_b128 %7, %15\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
            : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
            : "memory");
    }
#else
    for (int x = 0; x < N; ++x) r[x] = bf16x8{};
    (void)a;
#endif
}

// Eight 16-byte LDS reads at a + 64 jj + 16 h (jj < 4, h < 2; r[2 jj + h]): the
// per-row pairs (statistics or query descriptors) of one wave half's 16 rows.
__device__ __forceinline__ void lds_read_pairs(f32x4 (&r)[8], unsigned a)
{
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:16\n\t"
        "ds_read_b128 %2, %8 offset:64\n\t"
        "ds_read_b128 %3, %8 offset:80\n\t"
        "ds_read_b128 %4, %8 offset:128\n\t"
        "ds_read_b128 %5, %8 offset:144\n\t"
        "ds_read_b128 %6, %8 offset:192\n\t"
        "ds_read_b128 %7, %8 offset:208\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(a)
        : "memory");
#else
    for (int x = 0; x < 8; ++x) r[x] = f32x4{};
    (void)a;
#endif
}

// Sixteen bias entries of a strip, r[4 jj + e] at a + (8 jj + 2 e) * RUNB:
// 4-byte entries (fp32 profiles, RUNB 128) or 2-byte ones, zero-extended
// (bf16, RUNB 64).
template <bool PB>
__device__ __forceinline__ void lds_read_bias(unsigned (&r)[16], unsigned a)
{
#if defined(__HIP_DEVICE_COMPILE__)
    if constexpr (!PB) {
        asm volatile(
            "ds_read_b32 %0, %16\n\t"
            "ds_read_b32 %1, %16 offset:256\n\t"
            "ds_read_b32 %2, %16 offset:512\n\t"
            "ds_read_b32 %3, %16 offset:768\n\t"
            "ds_read_b32 %4, %16 offset:1024\n\t"
            "ds_read_b32 %5, %16 offset:1280\n\t"
            "ds_read_b32 %6, %16 offset:1536\n\t"
            "ds_read_b32 %7, %16 offset:1792\n\t"
            "ds_read_b32 %8, %16 offset:2048\n\t"
            "ds_read_b32 %9, %16 offset:2304\n\t"
            "ds_read_b32 %10, %16 offset:2560\n\t"
            "ds_read_b32 %11, %16 offset:2816\n\t"
            "ds_read_b32 %12, %16 offset:3072\n\t"
            "ds_read_b32 %13, %16 offset:3328\n\t"
            "ds_read_b32 %14, %16 offset:3584\n\t"
            "ds_read_b32 %15, %16 offset:3840\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
              "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15])
            : "v"(a)
            : "memory");
    } else {
        asm volatile(
            "ds_read_u16 %0, %16\n\t"
            "ds_read_u16 %1, %16 offset:128\n\t"
            "ds_read_u16 %2, %16 offset:256\n\t"
            "ds_read_u16 %3, %16 offset:384\n\t"
            "ds_read_u16 %4, %16 offset:512\n\t"
            "ds_read_u16 %5, %16 offset:640\n\t"
            "ds_read_u16 %6, %16 offset:768\n\t"
            "ds_read_u16 %7, %16 offset:896\n\t"
            "ds_read_u16 %8, %16 offset:1024\n\t"
            "ds_read_u16 %9, %16 offset:1152\n\t"
            "ds_read_u16 %10, %16 offset:1280\n\t"
            "ds_read_u16 %11, %16 offset:1408\n\t"
            "ds_read_u16 %12, %16 offset:1536\n\t"
            "ds_read_u16 %13, %16 offset:1664\n\t"
            "ds_read_u16 %14, %16 offset:1792\n\t"
            "ds_read_u16 %15, %16 offset:1920\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
              "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15])
            : "v"(a)
            : "memory");
    }
#else
    for (int x = 0; x < 16; ++x) r[x] = 0u;
    (void)a;
#endif
}

// Two 16-byte LDS reads at a and a + 1024.
__device__ __forceinline__ void lds_read_two(bf16x8& r0, bf16x8& r1, unsigned a)
{
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %2 offset:1024\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1)
        : "v"(a)
        : "memory");
#else
    r0 = bf16x8{};
    r1 = bf16x8{};
    (void)a;
#endif
}

// LDS byte address of a pointer into the workgroup's shared memory.
__device__ __forceinline__ unsigned lds_addr(const void* p)
{
    return (unsigned)(size_t)(const __attribute__((address_space(3))) char*)p;
}

// One LDS DMA (buffer_load ... lds) of SIZE bytes per lane (16, 4 or 2) from
// the buffer rsrc at the lane's byte offset voff into the LDS from byte lds
// on (lane l at lds + SIZE l), in an asm block: the compiler does not see an
// LDS write it cannot place, so it adds no wait for it before later LDS reads
// or writes of registers (through the builtin it waited for every DMA in
// flight there).  Every read of DMA'd data follows an explicit vmcnt wait and
// a barrier; the compiler's own vmcnt counts only grow stricter with DMAs it
// does not count (they complete in order).  The compiler's hazard pass does
// not look inside the block, so it begins with the wait states its sources
// may need: one after the M0 write the compiler puts right before it, five
// after a VALU write of an SGPR it reads (v_readlane restoring a spilled
// buffer resource, for one).
template <int SIZE>
__device__ __forceinline__ void dma_to_lds(__amdgpu_buffer_rsrc_t rsrc, unsigned lds, unsigned voff)
{
    static_assert(SIZE == 16 || SIZE == 4 || SIZE == 2, "16, 4 or 2 bytes per lane");
#if defined(__HIP_DEVICE_COMPILE__)
    const unsigned m = __builtin_amdgcn_readfirstlane(lds);
    if constexpr (SIZE == 16)
        asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" :: "v"(voff), "s"(rsrc), "{m0}"(m) : "memory");
    else if constexpr (SIZE == 4)
        asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds" :: "v"(voff), "s"(rsrc), "{m0}"(m) : "memory");
    else
        asm volatile("s_nop 4\n\tbuffer_load_ushort %0, %1, 0 offen lds" :: "v"(voff), "s"(rsrc), "{m0}"(m) : "memory");
#else
    (void)rsrc; (void)lds; (void)voff;
#endif
}

// ---------------------------------------------------------------------------
// dQ and the profile gradients.  One workgroup of 8 waves per (batch row, K/V
// head, head chunk, group of 32-query blocks), the forward's decomposition
// into 4 units (query head, 32-query block).  Wave w takes unit w % 4 and the
// 32-key half w / 4 of every key tile (two waves per SIMD); the two halves'
// dQ partials are summed at the end.  Lane = (query qi, wave half hh).
// ---------------------------------------------------------------------------
template <int D, bool PB>
__global__ __launch_bounds__(64 * DQ_WAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdParams p)
{
    constexpr int NW = DQ_WAVES;
    constexpr int NU = BW_WAVES;
    constexpr int NKK = D / 16;              // k-steps over D
    constexpr int NDB = D / 32;              // 32-row blocks of dQ^T
    constexpr int CH = D / 8;                // 16-byte chunks per row
    constexpr int TBYTES = BN * D * 2;       // one K or V tile
    constexpr int K_OFF = 0, V_OFF = TBYTES, CA_OFF = 2 * TBYTES;
    constexpr int STAGE = 2 * TBYTES + BN * 4;
    constexpr int NSCHED = 64 * NW;
    // per-wave bias strips (16 values per lane), two per wave: the tiles of
    // even and odd schedule position
    constexpr int B_OFF = 2 * STAGE;
    constexpr int BSW = 32 * 32 * 4;         // one wave's strip
    constexpr int SCHED_OFF = B_OFF + 2 * NW * BSW;
    static_assert(NU * (D / 32) * 16 * 64 * 4 <= B_OFF + 2 * NW * BSW,
                  "the dQ partials fit the staging buffers and strips");
    constexpr int LDS_BYTES = SCHED_OFF + (NSCHED + NW) * 4;
    constexpr int GPW = TBYTES / 1024 / NW;  // 1 KB DMA groups per wave of one K or V tile
    constexpr int RPG = 1024 / (2 * D);      // K / V rows per DMA group
    static_assert(GPW >= 1 && TBYTES % (1024 * NW) == 0, "tile DMA groups must divide among the waves");

    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int unit = wave % NU, kh = wave / NU;   // unit; key half (keys 32 kh .. 32 kh + 31 of a tile)
    const int qi = lane & 31, hh = lane >> 5;

    int idx = blockIdx.x;
    const int ngroups = p.Hkv * p.nchunk;
    const int hgi = idx % ngroups; idx /= ngroups;
    const int b = idx % p.B; idx /= p.B;
    const int qg = p.nQG - 1 - idx;
    const int g = hgi / p.nchunk;
    const int h = g * p.G + (hgi - g * p.nchunk) * p.hpw + unit % p.hpw;
    const int qb = qg * p.tpw + unit / p.hpw;
    const int qb_first = qg * p.tpw;
    const int qb_last = min(p.nQB - 1, qb_first + p.tpw - 1);
    const int i0 = qb * BM;
    const int i = i0 + qi;
    const bool qin = qb < p.nQB && i < p.Sq;
    const int gi = p.qoff + i;
    const unsigned wlim = p.window > 0 ? (unsigned)p.window : 0x80000000u;

    int2 qinf = make_int2(-1, 0);
    float2 rs = make_float2(0.0f, 0.0f);
    bf16x8 qreg[NKK], doreg[NKK];
    {
        const long long ro = (((long long)b * p.Sq + i) * p.Hq + h) * D + 8 * hh;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            qreg[kk] = qin ? *(const bf16x8*)(p.q + ro + 16 * kk) : bf16x8{};
            doreg[kk] = qin ? *(const bf16x8*)(p.dob + ro + 16 * kk) : bf16x8{};
        }
        if (qin) {
            qinf = p.qinfo[(size_t)b * p.Sq + i];
            rs = p.rowstat[((size_t)b * p.Hq + h) * p.Sq + i];
        }
    }
    const int gi_eff = qinf.x, a_q = qinf.y;
    if (qinf.x < 0) {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) qreg[kk] = bf16x8{};
    }
    const float lse2 = rs.x, dlt = rs.y;
    const size_t prow_off = (((size_t)b * p.Hq + h) * p.Sq + (qin ? i : 0)) * (size_t)p.E;
    char* const dprow = (char*)p.dprofiles + prow_off * (PB ? 2 : 4);

    f32x16 dqacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dqacc[db] = f32x16{};

    // ---- key-tile range of the workgroup (as the forward's)
    int jlo = INT_MAX, jhi = -1;
    for (int x = qb_first; x <= qb_last; ++x) {
        const TileSummary s = p.qsum[(size_t)b * p.nQB + x];
        if (s.nvalid == 0) continue;
        const int xlo = p.qoff + x * BM;
        const int xhi = p.qoff + min(p.Sq, x * BM + BM) - 1;
        int lo = max(0, s.amin);
        if (p.window > 0) lo = max(lo, xlo - p.window + 1);
        jlo = min(jlo, lo);
        jhi = max(jhi, min(p.Sk - 1, xhi));
    }
    // (workgroup-uniform; loaded with vector loads, hence the readfirstlane)
    const int kt_lo = __builtin_amdgcn_readfirstlane(jhi >= 0 ? jlo / BN : 0);
    const int kt_hi = __builtin_amdgcn_readfirstlane(jhi >= 0 ? jhi / BN : -1);
    // class of tile kt against block x (0 skip / 1 masked / 2 full) in bits 2 (x - qb_first)
    auto classify = [&](int kt) -> int {
        if (kt > kt_hi) return -1;
        const int j0 = kt * BN;
        const int kcount = min(BN, p.Sk - j0);
        const TileSummary ks = p.ksum[(size_t)b * p.nKT + kt];
        int code = 0;
        for (int x = qb_first; x <= qb_last; ++x) {
            const TileSummary qs = p.qsum[(size_t)b * p.nQB + x];
            const int xc = min(BM, p.Sq - x * BM);
            const int xlo = p.qoff + x * BM;
            code |= classify_tile(qs, xlo, xlo + xc - 1, xc, ks, j0, j0 + kcount - 1, kcount, p.window)
                    << (2 * (x - qb_first));
        }
        return code;
    };
    Schedule<NSCHED> sch;
    sch.list = (int*)(smem + SCHED_OFF);
    sch.base = kt_lo;
    sch.n = 0;
    sch.i = 0;

    // ---- staging.  Every global load of a tile is a buffer load issued at
    // the start of the iteration before and stored to LDS at its end, so the
    // loads have a whole iteration to land.  Rows past Sk read as 0.
    const unsigned krow = (unsigned)(p.Hkv * D * 2);          // bytes between consecutive keys
    const unsigned knrec = p.Sk > 0 ? (unsigned)(p.Sk - 1) * krow + D * 2 : 0u;
    const long long kvbase = ((long long)b * p.Sk * p.Hkv + g) * D;
    const __amdgpu_buffer_rsrc_t krs = uniform_rsrc(p.k + kvbase, knrec);
    const __amdgpu_buffer_rsrc_t vrs = uniform_rsrc(p.v + kvbase, knrec);
    const __amdgpu_buffer_rsrc_t kas = uniform_rsrc(p.kanchor + (size_t)b * p.nKT * BN, (size_t)p.nKT * BN * 4);
    constexpr int ES = PB ? 2 : 4;                               // profile element bytes
    const size_t pblock = (size_t)p.Sq * p.E * ES;               // one (batch row, head) of profiles
    const __amdgpu_buffer_rsrc_t prs =
        uniform_rsrc((const char*)p.profiles + ((size_t)b * p.Hq + h) * pblock, pblock);
    const __amdgpu_buffer_rsrc_t drs = uniform_rsrc((char*)p.dprofiles + ((size_t)b * p.Hq + h) * pblock, pblock);
    const unsigned rowe = (unsigned)(qin ? i : 0) * (unsigned)p.E;   // this query's row, in entries
    // Bias class of a tile for this wave: no distance of its 32 x 32 pairs
    // (its key half) in [0, E) (no bias, no profile gradient), all inside
    // (whole 16-byte runs), or mixed (entry by entry).  Wave-uniform.
    const int qlo_w = p.qoff + i0, qhi_w = p.qoff + min(p.Sq, i0 + BM) - 1;
    auto bias_class = [&](int j0t) -> int {
        if (qb >= p.nQB) return BC_NONE;
        const int jh = j0t + 32 * kh;
        const int rmin = qlo_w - (jh + 31), rmax = qhi_w - jh;
        if (rmax < 0 || rmin >= p.E) return BC_NONE;
        return (rmin >= 0 && rmax < p.E) ? BC_FULL : BC_EDGE;
    };
    // tiles before kt_split carry no bias for any wave of the workgroup (every
    // distance of its first query column to the tile's last key is at least E)
    const int qlo_wg = p.qoff + qb_first * BM;
    const int kt_split = p.E <= 0 ? INT_MAX : (qlo_wg - p.E - (BN - 1) >= 0 ? (qlo_wg - p.E - (BN - 1)) / BN + 1 : 0);
    // K, V and the key start columns of tile kt go to stage buffer sb by
    // buffer -> LDS DMA: lane l of 1 KB group a writes bytes 1024 a + 16 l of
    // the tile and fetches the chunk that belongs there (row RPG a + l / CH,
    // slot l % CH, i.e. chunk slot ^ row_swz(row)).  Every wave also fetches
    // the same 64 start columns, so that each wave's sequence of memory
    // instructions is the same on every path.
    // The lane's part of the offset (row RPG wave + ln / CH of the tile, its
    // chunk) is formed once: group a = wave + NW u adds RPG NW u rows, which
    // leaves the row's swizzle (a function of the row modulo 16) unchanged.
    static_assert(GPW == 1 || (RPG * NW) % 16 == 0, "the swizzle of a lane's rows is the same in every group");
    const unsigned kvlane = [&] {
        const unsigned r = (unsigned)(RPG * wave) + (unsigned)lane / CH;
        return opaque(r * krow + 16u * (((unsigned)lane % CH) ^ (unsigned)row_swz<D>((int)r)));
    }();
    auto stage_load = [&](int kt, int sb) {
        const int j0 = kt * BN;
        char* const st = smem + sb * STAGE;
#pragma unroll
        for (int u = 0; u < GPW; ++u) {
            const int a = wave + NW * u;
            // (whole offsets in the register operand: the range check, which
            // turns rows past Sk into zeros, applies to it)
            const unsigned kvo = kvlane + (unsigned)(j0 + RPG * NW * u) * krow;
            dma_to_lds<16>(krs, lds_addr(st + K_OFF + 1024 * a), kvo);
            dma_to_lds<16>(vrs, lds_addr(st + V_OFF + 1024 * a), kvo);
        }
        const unsigned cao = (unsigned)j0 * 4u + 4u * opaque((unsigned)lane);
        dma_to_lds<4>(kas, lds_addr(st + CA_OFF), cao);
    };
    // This wave's bias of tile kt goes by DMA into a strip of the wave, about
    // two tiles ahead of its use.  Entry (jj, e) of a lane is distance rb + e
    // with rb = gi - (j0 + 32 kh + 8 jj + 4 hh + 3).  Whole runs (BC_FULL,
    // fp32): row qi of the wave's 32 x 32 block needs the 32 distances from
    // gi - (j0 + 32 kh + 31) up, 128 contiguous bytes of its profile row; the
    // strip holds them row-major (128 bytes per row), its 16-byte chunk c at
    // slot c ^ run_swz(qi), and one instruction fetches 8 whole rows (lane l
    // of instruction a: row 8 a + l / 8, slot l % 8), so that every request
    // covers whole runs of a row rather than 32 bytes of each of 32 rows.
    // Otherwise one entry per instruction, lane-major per (jj, e) (bytes
    // 256 (4 jj + e) + 4 l; a bf16 entry lands zero-extended in its dword).
    // Returns the class; the instructions issued are bias_dmas(class).
    // Byte offset, in the profile (or gradient) block of the head, of the 16
    // bytes that lane ln moves in whole-run instruction a of the tile at key
    // column j0: row r = 8 a + ln / 8 of the wave's block, its run chunk
    // (ln % 8) ^ run_swz(r); past the buffer (dropped) for rows past Sq.
    auto run_off = [&](unsigned ln, int a, int j0t) -> unsigned {
        const unsigned r = 8u * (unsigned)a + ln / 8u;
        const unsigned c = (ln % 8u) ^ run_swz(r);
        const int row = i0 + (int)r;
        const unsigned d0 = (unsigned)(p.qoff + row - (j0t + 32 * kh + 31));   // the run's first distance
        return row < p.Sq ? ((unsigned)row * (unsigned)p.E + d0) * 4u + 16u * c : 0xFFFFFFF0u;
    };
    auto bias_dma = [&](int kt, char* strip) -> int {
        if (kt < 0 || kt < kt_split) return BC_NONE;
        const int j0 = kt * BN;
        const int bc = bias_class(j0);
        if (bc == BC_NONE) return BC_NONE;
        lds_char* const sp = opaque_lds((lds_char*)strip);
        const unsigned ln = opaque((unsigned)lane);
        if (!PB && bc == BC_FULL) {
#pragma unroll
            for (int a = 0; a < 4; ++a)
                dma_to_lds<16>(prs, (unsigned)(size_t)(sp + 1024 * a), run_off(ln, a, j0));
            return bc;
        }
        const unsigned gb = (unsigned)gi - (unsigned)(j0 + 32 * kh + 3) - 4u * (ln >> 5);   // rb + 8 jj
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            // (entry offsets kept opaque: they may wrap modulo 2^32 like the run's start)
            const unsigned off = (rowe + gb - 8u * (unsigned)jj) * (unsigned)ES;
            {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (PB)
                        dma_to_lds<2>(prs, (unsigned)(size_t)(sp + 256 * (4 * jj + e)), opaque(off + 2u * e));
                    else
                        dma_to_lds<4>(prs, (unsigned)(size_t)(sp + 256 * (4 * jj + e)), opaque(off + 4u * e));
                }
            }
        }
        return bc;
    };
    auto bias_dmas = [&](int bc) -> int { return bc == BC_NONE ? 0 : (!PB && bc == BC_FULL) ? 4 : 16; };
    // profile-gradient stores of a tile of class bc (see the body)
    auto grad_stores = [&](int bc) -> int { return bc == BC_NONE ? 0 : (!PB && bc == BC_FULL) ? 4 : 16; };
    char* const bstrip0 = smem + B_OFF + wave * BSW;   // strip 0 of this wave; strip 1 at + NW * BSW

    using F = std::false_type;
    using T = std::true_type;
    // While the current tile lies before kt_split, a loop body without the
    // bias code runs.
    int2 cur = next_entry(sch, kt_hi, classify);
    int2 nxt = make_int2(-1, 0), nx2 = make_int2(-1, 0);
    int par = 0;        // strip of cur: its position in the schedule, mod 2
    if (cur.x >= 0) {
        stage_load(cur.x, 0);
        bias_dma(cur.x, bstrip0);
        nxt = next_entry(sch, kt_hi, classify);
        bias_dma(nxt.x, bstrip0 + NW * BSW);
        if (nxt.x >= 0) nx2 = next_entry(sch, kt_hi, classify);
    }
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_s_waitcnt(0);   // nothing loaded before the loop is outstanding inside it
#endif
    __syncthreads();
    int buf = 0;
    const int xw = qb - qb_first;
    const float nlse2 = -lse2;
    // K^T operand of dQ^T += K^T dS^T, from the K rows by transposing LDS
    // reads: for 16-key step c and d-block db, lane l reads 4 bf16 of key row
    // 16 c + 4 hh + (l % 16) / 4 (and 8 rows further) at columns 32 db +
    // 16 ((l / 16) % 2) + 4 (l % 4), and receives column d = 32 db + (l % 32)
    // of the keys 16 c + 4 hh + t and 16 c + 8 + 4 hh + t, t < 4: the order of
    // the dS^T operand below.  trof() is the byte offset in the swizzled rows
    // (formed where used: not held in registers across the loop); for D = 128
    // one base per lane serves every read (tr_base128).
    static_assert(D != 128 || STAGE % 256 == 0, "stage rows start on 256-byte boundaries");
    const unsigned trb = D == 128 ? opaque(tr_base128((unsigned)lane) + 8192u * (unsigned)kh) : 0u;
    auto trof = [&](unsigned ln, int c2, int hi, int db) -> unsigned {
        const unsigned r = 16u * (unsigned)(2 * kh + c2) + 8u * (unsigned)hi + 4u * (ln >> 5) + (ln & 15u) / 4u;
        const unsigned col = 32u * (unsigned)db + 16u * ((ln >> 4) & 1u) + 4u * (ln & 3u);   // bf16 column
        return (unsigned)K_OFF + r * (2u * D) + 16u * ((col / 8u) ^ (unsigned)row_swz<D>((int)r)) + 2u * (col % 8u);
    };
    auto step = [&](auto with_bias) {
        constexpr bool WB = decltype(with_bias)::value;
        const int j0 = cur.x * BN;
        const int my_cls = (cur.y >> (2 * xw)) & 3;
        const int bc = WB ? bias_class(j0) : (int)BC_NONE;
        const char* st = smem + buf * STAGE;
        char* const strip = bstrip0 + par * (NW * BSW);
        // ---- this tile's bias out of its strip (it landed by the end of the
        // iteration before); entries (jj, 0..3) of a whole run are chunk
        // 7 - 2 jj - hh of row qi
        f32x4 bv[4];
        const unsigned rslot = 128u * (unsigned)qi + 16u * ((7u - (unsigned)hh) ^ run_swz((unsigned)qi));
        if constexpr (WB) {
            if (bc != BC_NONE) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    if (!PB && bc == BC_FULL) {
                        bv[jj] = *(const f32x4*)(strip + (rslot ^ (32u * (unsigned)jj)));
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const unsigned x = *(const unsigned*)(strip + 256 * (4 * jj + e) + 4 * lane);
                            bv[jj][e] = PB ? __uint_as_float(x << 16) : __uint_as_float(x);
                        }
                    }
                }
            }
        }
        asm volatile("" ::: "memory");
        // (buffer buf ^ 1 was last read before the barrier that ended the
        // previous iteration)
        if (nxt.x >= 0) stage_load(nxt.x, buf ^ 1);
        asm volatile("" ::: "memory");

        // ---- S^T = K Q^T and dP^T = V dO^T for this wave's key half, keys
        // 32 kh + ((lane & 31) ^ 3) on M
        // (the operands of k-step kk + 1 are read while k-step kk multiplies)
        f32x16 acc = f32x16{}, dacc = f32x16{};
        {
            const int r = 32 * kh + (qi ^ 3);
            auto opnd = [&](int kk, int off) -> bf16x8 {
                return *(const bf16x8*)(st + off + r * (2 * D) + 16 * ((2 * kk + hh) ^ row_swz<D>(r)));
            };
            bf16x8 ak[2], av[2];
            ak[0] = opnd(0, K_OFF);
            av[0] = opnd(0, V_OFF);
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                if (kk + 1 < NKK) {
                    ak[(kk + 1) & 1] = opnd(kk + 1, K_OFF);
                    av[(kk + 1) & 1] = opnd(kk + 1, V_OFF);
                }
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[kk & 1], qreg[kk], acc, 0, 0, 0);
                dacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[kk & 1], doreg[kk], dacc, 0, 0, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);       // LDS reads
#pragma unroll
            for (int kk = 0; kk + 1 < NKK; ++kk) {
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // LDS reads
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);       // MFMA
        }

        // ---- P, dS, profile gradients.  Element (jj, e) is key
        // j0 + 32 kh + 8 jj + 4 hh + (e ^ 3), distance rb + e with
        // rb = gi - (j0 + 32 kh + 8 jj + 4 hh + 3).  The dS^T operand holds the
        // keys of each group of 4 in increasing order (element 4 (jj % 2) + (e ^ 3)).
        const int* ca = (const int*)(st + CA_OFF);
        bf16x8 pd[2];
        auto body = [&](auto bct, auto mt) {
            constexpr int BCT = decltype(bct)::value;
            constexpr bool MASKED = decltype(mt)::value;
            {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int kl = 32 * kh + 8 * jj + 4 * hh;
                    const int rb = gi - (j0 + kl + 3);
                    f32x4 pre;   // bias * log2(e) - lse2 per entry
                    if constexpr (BCT == BC_NONE) {
                        pre = f32x4{nlse2, nlse2, nlse2, nlse2};
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            pre[e] = __builtin_fmaf(bv[jj][e], LOG2E, nlse2);
                            if constexpr (BCT == BC_EDGE)
                                if ((unsigned)(rb + e) >= (unsigned)p.E) pre[e] = nlse2;
                        }
                    }
                    i32x4 c4;
                    if constexpr (MASKED) c4 = *(const i32x4*)(ca + kl);
                    f32x4 dz;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[4 * jj + e], p.c_log2, pre[e]));
                        const float x = pr * (dacc[4 * jj + e] - dlt);
                        if constexpr (MASKED)   // (keys that are not real may hold any value)
                            dz[e] = key_visible(gi_eff, a_q, j0 + kl + (e ^ 3), c4[e ^ 3], wlim) ? x : 0.0f;
                        else
                            dz[e] = x;
                        pd[jj >> 1][4 * (jj & 1) + (e ^ 3)] = (__bf16)dz[e];
                    }
                    // profile gradients: stores outside this query's row [0, E)
                    // get an offset past the buffer and are dropped
                    if constexpr (BCT == BC_FULL) {
                        if constexpr (PB) {
                            const unsigned off = qin ? (rowe + (unsigned)rb) * (unsigned)ES : 0xFFFFFFF0u;
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                __builtin_amdgcn_raw_buffer_store_b16(
                                    (unsigned short)(__float_as_uint((float)(__bf16)dz[e]) >> 16), drs,
                                    opaque(off + 2u * e), 0, 0);
                        } else {
                            // into the strip, in the whole-run layout of the bias
                            // (its entries were read at the start of the step)
                            *(f32x4*)(strip + (rslot ^ (32u * (unsigned)jj))) = dz;
                        }
                    } else if constexpr (BCT == BC_EDGE) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const bool inside = qin && (unsigned)(rb + e) < (unsigned)p.E;
                            const unsigned off = inside ? (rowe + (unsigned)(rb + e)) * (unsigned)ES : 0xFFFFFFF0u;
                            if constexpr (PB)
                                __builtin_amdgcn_raw_buffer_store_b16(
                                    (unsigned short)(__float_as_uint((float)(__bf16)dz[e]) >> 16), drs, off, 0, 0);
                            else
                                __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(dz[e]), drs, off, 0, 0);
                        }
                    }
                }
                if constexpr (BCT == BC_FULL && !PB) {
                    // whole runs back out of the strip, 8 rows per store (the
                    // wave's own LDS writes above precede these reads)
                    const unsigned ln = opaque((unsigned)lane);
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const f32x4 w = *(const f32x4*)(strip + 1024 * a + 16 * lane);
                        __builtin_amdgcn_raw_buffer_store_b128(
                            i32x4{__float_as_int(w[0]), __float_as_int(w[1]), __float_as_int(w[2]),
                                  __float_as_int(w[3])},
                            drs, run_off(ln, a, j0), 0, 0);
                    }
                }
            }
        };
        using NONE = std::integral_constant<int, BC_NONE>;
        using FULL = std::integral_constant<int, BC_FULL>;
        using EDGE = std::integral_constant<int, BC_EDGE>;
        if constexpr (!WB) {
            if (my_cls == TILE_FULL) body(NONE{}, F{});
            else body(NONE{}, T{});
        } else if (my_cls == TILE_FULL) {
            if (bc == BC_NONE) body(NONE{}, F{});
            else if (bc == BC_FULL) body(FULL{}, F{});
            else body(EDGE{}, F{});
        } else {
            if (bc == BC_NONE) body(NONE{}, T{});
            else if (bc == BC_FULL) body(FULL{}, T{});
            else body(EDGE{}, T{});
        }
        asm volatile("" ::: "memory");
        // the strip takes the bias of the tile two ahead (this tile's entries
        // and gradients are out of it: the stores above took their data)
        const int nbc2 = bias_dma(nx2.x, strip);
        asm volatile("" ::: "memory");

        // ---- dQ^T += K^T dS^T over this wave's key half (16-key steps
        // 2 kh, 2 kh + 1), K^T read from the K rows
        const unsigned tln = opaque((unsigned)lane);
        const unsigned stl = lds_addr(st);
        unsigned ad128[2 * NDB];   // D = 128: the reads of 16-key step 0 (step 1 at + 4096)
        if constexpr (D == 128) {
            const unsigned x0 = stl + trb;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                ad128[2 * db] = x0 ^ (64u * (unsigned)db);
                ad128[2 * db + 1] = (x0 + 2048u) ^ (64u * (unsigned)db + 32u);
            }
        }
        auto dq_part = [&](auto c2v) {
            constexpr int c2 = decltype(c2v)::value;
            s16x4 rd[2 * NDB];
            if constexpr (D == 128) {
                tr_read<2 * NDB, 4096 * c2>(rd, ad128);
            } else {
                unsigned ad[2 * NDB];
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    ad[2 * db] = stl + trof(tln, c2, 0, db);
                    ad[2 * db + 1] = stl + trof(tln, c2, 1, db);
                }
                tr_read<2 * NDB>(rd, ad);
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const s16x8 a8 = __builtin_shufflevector(rd[2 * db], rd[2 * db + 1], 0, 1, 2, 3, 4, 5, 6, 7);
                dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a8), pd[c2],
                                                                   dqacc[db], 0, 0, 0);
            }
        };
        dq_part(std::integral_constant<int, 0>{});
        dq_part(std::integral_constant<int, 1>{});

        // this wave's DMA of the next tile has landed (the bias DMA of the
        // tile two ahead and this tile's profile-gradient stores, issued after
        // it, may still be in flight); then every wave's has
        wait_vm_and_barrier(bias_dmas(nbc2) + (WB ? grad_stores(bc) : 0));
        buf ^= 1;
        par ^= 1;
        cur = nxt;
        nxt = nx2;
        nx2 = nxt.x >= 0 ? next_entry(sch, kt_hi, classify) : make_int2(-1, 0);
    };
    while (cur.x >= 0 && cur.x < kt_split) step(F{});
    while (cur.x >= 0) step(T{});

    // ---- the two key halves' partials (the staging buffers are free: the
    // last iteration ended at a barrier): half 1 hands its partial to half 0
    // through LDS, then writes the profile-gradient zeros while half 0 writes dq
    {
        float* red = (float*)smem + (size_t)unit * NDB * 16 * 64 + lane;
        if (kh == 1) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int t = 0; t < 16; ++t) red[(db * 16 + t) * 64] = dqacc[db][t];
        }
        __syncthreads();
        if (kh == 0) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int t = 0; t < 16; ++t) dqacc[db][t] += red[(db * 16 + t) * 64];
        }
    }
    if (!qin) return;
    // ---- dq = scale * dQ^T
    if (kh == 0) {
        float* dqp = p.dq + (((size_t)b * p.Sq + i) * p.Hq + h) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                f32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = dqacc[db][4 * jj + e] * p.scale;
                *(f32x4*)(dqp + 32 * db + 8 * jj + 4 * hh) = w;
            }
    }

    if (kh == 0) return;
    // ---- zeros at the profile-gradient entries no visited tile wrote: the
    // distance r belongs to key column gi - r, so these are the columns
    // outside [0, Sk) and those in tiles the workgroup did not visit.
    // Each half of the wave takes every other run of 4 distances.
    auto zero_range = [&](int rlo, int rhi) {   // distances rlo .. rhi of this lane's row
        rlo = max(rlo, 0);
        rhi = min(rhi, p.E - 1);
        for (int r = rlo + 4 * hh; r <= rhi; r += 8)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (r + e <= rhi) store_grad<PB>(dprow, r + e, 0.0f);
    };
    zero_range(gi + 1, p.E - 1);                      // columns below 0
    zero_range(0, gi - p.Sk);                         // columns at or past Sk
    const int wlo_col = p.qoff + qb_first * BM - p.E + 1;
    const int whi_col = min(p.Sk - 1, p.qoff + min(p.Sq, (qb_last + 1) * BM) - 1);
    if (whi_col >= 0) {
        for (int kt = max(0, wlo_col) / BN; kt <= whi_col / BN; ++kt) {
            const int code = (kt >= kt_lo && kt <= kt_hi) ? classify(kt) : 0;
            if (code > 0) continue;                   // visited: every entry written
            zero_range(gi - (kt * BN + BN - 1), gi - kt * BN);
        }
    }
}

// ---------------------------------------------------------------------------
// dK and dV.  One workgroup of 8 waves per (batch row, K/V head, 128 keys);
// two waves share each 32-key group (on one SIMD): the P wave (waves 0..3)
// holds K, computes S = Q K^T and P and accumulates dV^T += dO^T P; the dS
// wave (waves 4..7) holds V, computes dP = dO V^T, takes P from the P wave
// through LDS, forms dS and accumulates dK^T += Q^T dS.  Lane = (key kl,
// half hh).  The workgroup walks the live 32-query blocks (from the last
// down) and, for each, every query head of the group.
// ---------------------------------------------------------------------------
template <int D, bool PB>
__global__ __launch_bounds__(64 * KV_WAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(BwdParams p)
{
    constexpr int NW = KV_WAVES;
    constexpr int NKK = D / 16;
    constexpr int NDB = D / 32;
    constexpr int RBYTES = BM * D * 2;       // one 32-row Q / dO tile
    // one stage: Q rows, dO rows, row statistics, query descriptors, and the
    // P waves' bias strips; four stages in a ring, then the P exchange
    constexpr int Q_OFF = 0, DO_OFF = RBYTES;
    constexpr int RS_OFF = 2 * RBYTES, QI_OFF = RS_OFF + BM * 8;
    constexpr int BS_OFF = QI_OFF + BM * 8;
    constexpr int ES = PB ? 2 : 4;             // profile element bytes
    constexpr int BSW = 32 * 32 * ES;          // one key group's bias strip: 32 rows x 32 keys
    constexpr int STAGE = BS_OFF + 4 * BSW;
    constexpr int NBUF = 4;
    constexpr int XP_OFF = NBUF * STAGE;       // P of each key group, bf16 in register order (2 KB), two slots
    constexpr int NSCHED = 64 * NW;
    constexpr int SCHED_OFF = XP_OFF + 2 * 4 * 2048;
    constexpr int LDS_BYTES = SCHED_OFF + (NSCHED + NW) * 4;
    constexpr int NRI = RBYTES / 1024 / NW;    // 1 KB DMA instructions per wave and 32-row tile
    static_assert(NRI >= 1 || RBYTES == 1024 * 4, "");
    constexpr int NRT = RBYTES / 1024;         // 1 KB groups of a 32-row tile

    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = wave & 3, role = wave >> 2;   // key group; 0: P wave, 1: dS wave
    const int kl = lane & 31, hh = lane >> 5;

    int idx = blockIdx.x;
    const int g = idx % p.Hkv; idx /= p.Hkv;
    const int b = idx % p.B; idx /= p.B;
    const int kb = idx;                                // key blocks in increasing order
    const int jb0 = kb * KV_KEYS;
    const int jw = jb0 + 32 * kg;
    const int j = jw + kl;
    const bool kin = j < p.Sk;
    const int kt_first = jb0 / BN;
    const int kt_last = min(p.nKT - 1, kt_first + KV_KEYS / BN - 1);
    const int xk = (32 * kg) / BN;                     // this group's key tile within the block

    const int c_k = kin ? p.kanchor[(size_t)b * p.nKT * BN + j] : INT_MIN;
    const unsigned wlim = p.window > 0 ? (unsigned)p.window : 0x80000000u;
    // K (P waves) or V (dS waves) as the B operand: lane holds 8 d's of its key
    bf16x8 kvreg[NKK];
    {
        const bool ok = kin && c_k != INT_MIN;
        const __bf16* src = role ? p.v : p.k;
        const long long off = (((long long)b * p.Sk + j) * p.Hkv + g) * D + 8 * hh;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) kvreg[kk] = ok ? *(const bf16x8*)(src + off + 16 * kk) : bf16x8{};
    }
    f32x16 acc[NDB];   // dV^T (P waves) or dK^T (dS waves): rows d, column = key
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

    // ---- query-block range: causal (gi >= first key), window, document
    int qlo_col = INT_MAX, qhi_col = -1;
    for (int x = kt_first; x <= kt_last; ++x) {
        const TileSummary s = p.ksum[(size_t)b * p.nKT + x];
        if (s.nvalid == 0) continue;
        const int xlo = x * BN, xhi = min(p.Sk, x * BN + BN) - 1;
        qlo_col = min(qlo_col, xlo);
        int hi = p.qoff + p.Sq - 1;
        if (p.window > 0) hi = min(hi, xhi + p.window - 1);
        qhi_col = max(qhi_col, hi);
    }
    // (workgroup-uniform; loaded with vector loads, hence the readfirstlane)
    const int qb_lo = __builtin_amdgcn_readfirstlane(qhi_col >= 0 ? max(0, qlo_col - p.qoff) / BM : 0);
    const int qb_hi = __builtin_amdgcn_readfirstlane(
        (qhi_col >= 0 && qhi_col >= p.qoff) ? min(p.nQB - 1, (qhi_col - p.qoff) / BM) : -1);
    // Query blocks are walked from the last down to the first, so that the
    // workgroups on one XCD (one K/V head) stream the same query tiles at
    // about the same time and share them in L2: without a window every range
    // ends at the last block (or its document's), candidate c is block
    // qb_hi - c.  With a window the ranges end at different blocks, so the
    // descending walk is rotated to start at the block congruent to nQB - 1
    // modulo the range's length: workgroups whose ranges have one length
    // (every key block away from the sequence's ends) then meet each shared
    // block at the same candidate.
    const int nblk = qb_hi - qb_lo + 1;
    const int rot = (p.window > 0 && nblk > 0) ? (p.nQB - 1 - qb_lo) % nblk : nblk - 1;
    auto blk = [&](int c) -> int {   // c in [0, nblk)
        const int t = rot - c;
        return qb_lo + (t >= 0 ? t : t + nblk);
    };
    auto classify = [&](int c) -> int {
        if (c >= nblk) return -1;
        const int x = blk(c);
        const TileSummary qs = p.qsum[(size_t)b * p.nQB + x];
        const int xc = min(BM, p.Sq - x * BM);
        const int xlo = p.qoff + x * BM;
        int code = 0;
        for (int t = kt_first; t <= kt_last; ++t) {
            const int j0 = t * BN;
            const int kcount = min(BN, p.Sk - j0);
            const TileSummary ks = p.ksum[(size_t)b * p.nKT + t];
            code |= classify_tile(qs, xlo, xlo + xc - 1, xc, ks, j0, j0 + kcount - 1, kcount, p.window)
                    << (2 * (t - kt_first));
        }
        return code;
    };
    Schedule<NSCHED> sch;
    sch.list = (int*)(smem + SCHED_OFF);
    sch.base = 0;
    sch.n = 0;
    sch.i = 0;

    // ---- staging by LDS DMA (buffer_load ... lds) into a ring of four
    // stages: the stage of iteration t + 2 is requested in iteration t.  A
    // wave waits until at most the DMA instructions of the last stage it
    // requested are outstanding: the stage before has then landed.
    const unsigned qrow = (unsigned)(p.Hq * D * 2);            // bytes between consecutive queries
    const unsigned qnrec = (unsigned)(p.Sq - 1) * qrow + D * 2;
    const long long qbase = (long long)b * p.Sq * p.Hq * D;
    const size_t pblock = (size_t)p.Sq * p.E * ES;
    // Q / dO rows: 1 KB group a holds rows RPI a .. RPI a + RPI - 1; wave w
    // takes group w of each tile (groups past NRT: none); lane -> (row, LDS
    // chunk slot), it fetches the chunk that lands there
    constexpr int CPR = D / 8, RPI = 1024 / (2 * D);
    const bool has_rows = wave < NRT;
    unsigned qv;
    {
        const int a = has_rows ? wave : 0;
        const int r = RPI * a + lane / CPR, pc = lane % CPR;
        qv = (unsigned)r * qrow + 16u * (unsigned)(pc ^ row_swz<D>(r));
    }
    // Bias strip of a key group: for each of its 32 rows the run of 32
    // distances of its keys, qoff + i - (jw + 31) .. qoff + i - jw (key jw + kl
    // at entry 31 - kl).  Row m = 8 jj + 4 hh + e sits at slot 8 jj + 2 e + hh,
    // so the two wave halves read adjacent slots.
    constexpr int RUNB = 32 * ES;                // bytes of one run
    constexpr int PPR = RUNB / 16;               // 16-byte pieces per run
    constexpr int RSL = 64 / PPR;                // slots per DMA instruction
    constexpr int NBI = 32 / RSL;                // bias DMA instructions of a P wave
    unsigned bvo[NBI];
#pragma unroll
    for (int k = 0; k < NBI; ++k) {
        const int slot = RSL * k + lane / PPR, piece = lane % PPR;
        const int m = 8 * (slot / 8) + 4 * (slot & 1) + (slot % 8) / 2;
        bvo[k] = (unsigned)m * (unsigned)(p.E + 1) * (unsigned)ES + 16u * (unsigned)piece;
    }
    // bias class of a block for a key group (wave-uniform)
    auto bias_class = [&](int x) -> int {
        const int rmin = p.qoff + x * BM - (jw + 31), rmax = p.qoff + x * BM + BM - 1 - jw;
        if (rmax < 0 || rmin >= p.E) return BC_NONE;
        return (rmin >= 0 && rmax < p.E && x * BM + BM <= p.Sq) ? BC_FULL : BC_EDGE;
    };
    // Issues this wave's DMA of one stage; returns the number of DMA
    // instructions (a P wave fetches no bias runs for a block without bias:
    // its strip is not read then).
    auto issue = [&](int x, int h, int buf) -> int {
        int n = 0;
        char* st = smem + buf * STAGE;
        const int i0 = x * BM;
        if (has_rows) {
            const __amdgpu_buffer_rsrc_t qrs = uniform_rsrc(p.q + qbase + (long long)h * D, qnrec);
            const __amdgpu_buffer_rsrc_t drs = uniform_rsrc(p.dob + qbase + (long long)h * D, qnrec);
            const unsigned vo = qv + (unsigned)i0 * qrow;
            dma_to_lds<16>(qrs, lds_addr(st + Q_OFF + 1024 * wave), vo);
            dma_to_lds<16>(drs, lds_addr(st + DO_OFF + 1024 * wave), vo);
            n += 2;
        }
        if (wave < 2) {
            // row statistics (wave 0) or query descriptors (wave 1): one dword
            // per lane, rows past Sq read as 0
            const __amdgpu_buffer_rsrc_t xrs =
                wave ? uniform_rsrc(p.qinfo + (size_t)b * p.Sq, (size_t)p.Sq * 8)
                     : uniform_rsrc(p.rowstat + ((size_t)b * p.Hq + h) * p.Sq, (size_t)p.Sq * 8);
            const unsigned vo = (unsigned)i0 * 8u + 4u * (unsigned)lane;
            dma_to_lds<4>(xrs, lds_addr(st + (wave ? QI_OFF : RS_OFF)), vo);
            n += 1;
        }
        if (role == 0 && bias_class(x) != BC_NONE) {
            // row i0 + m, run start qoff + i0 + m - jw - 31: entry offset
            // (i0 + m) E + qoff + i0 + m - jw - 31 = m (E + 1) + i0 (E + 1) + qoff - jw - 31
            const __amdgpu_buffer_rsrc_t prs =
                uniform_rsrc((const char*)p.profiles + ((size_t)b * p.Hq + h) * pblock, pblock);
            const unsigned base = ((unsigned)i0 * (unsigned)(p.E + 1) + (unsigned)(p.qoff - jw - 31)) * (unsigned)ES;
            char* bs = st + BS_OFF + kg * BSW;
#pragma unroll
            for (int k = 0; k < NBI; ++k) {
                const unsigned vo = opaque(base + bvo[k]);
                dma_to_lds<16>(prs, lds_addr(bs + 1024 * k), vo);
            }
            n += NBI;
        }
        return n;
    };
    // Transposing reads (ds_read_b64_tr_b16) of the row tiles give the A
    // operands of dV^T = dO^T P and dK^T = Q^T dS: for query step c and
    // d-block db, lane l reads 4 bf16 of row 16 c + 4 hh + (l % 16) / 4 (and 8
    // rows further) at columns 32 db + 16 ((l / 16) % 2) + 4 (l % 4), and
    // receives column d = 32 db + (l % 32) of the queries 16 c + 4 hh + t and
    // 16 c + 8 + 4 hh + t, t < 4: the order of the P / dS registers.  trof[]
    // are the byte offsets of the lane's 8 bytes in the swizzled rows.
    // (D = 128: one base per lane, tr_base128; the others kept per read)
    static_assert(D != 128 || (STAGE % 256 == 0 && DO_OFF % 256 == 0), "row tiles start on 256-byte boundaries");
    int trof[2][2][NDB];
    const unsigned trb = D == 128 ? opaque(tr_base128((unsigned)lane)) : 0u;
    if constexpr (D != 128) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int hi = 0; hi < 2; ++hi)
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const int r = 16 * c + 8 * hi + 4 * hh + (lane & 15) / 4;
                    const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);   // bf16 column
                    trof[c][hi][db] = r * (2 * D) + 16 * ((col / 8) ^ row_swz<D>(r)) + 2 * (col % 8);
                }
    }

    // iteration = (live query block, head of the group); descriptors of the
    // next two are kept for the DMA ahead
    struct It {
        int x, code, hs;   // x < 0: none
    };
    auto next_block = [&]() -> It {
        const int2 e = next_entry(sch, qb_hi - qb_lo, classify);
        It r;
        r.x = e.x >= 0 ? blk(e.x) : -1;
        r.code = e.y;
        r.hs = 0;
        return r;
    };
    auto succ = [&](It d) -> It {
        if (d.x < 0) return d;
        if (d.hs + 1 < p.G) {
            d.hs += 1;
            return d;
        }
        return next_block();
    };
    // The dS wave runs one iteration behind its P wave: in iteration t the P
    // wave forms P of (block, head) t from stage t and the dS wave uses P of
    // t - 1 (exchange slot (t - 1) % 2) with stage t - 1, so the two need no
    // barrier between them; a last iteration drains the dS waves.  Stages:
    // t - 1 and t in use, t + 1 in flight, t + 2 requested: a ring of four.
    It cur = next_block();
    It n1 = succ(cur);
    It prv;
    prv.x = -1;
    prv.code = 0;
    prv.hs = 0;
    // The loop, specialised per role (each wave runs one of the two copies,
    // so neither carries the other's registers and branches).
    auto kv_loop = [&](auto rolec) {
        constexpr int ROLE = decltype(rolec)::value;
        int n_flight = 0;   // DMA instructions of the last stage requested
#if defined(__HIP_DEVICE_COMPILE__)
        // the K / V operands and the other loads above have landed: the compiler
        // then keeps no wait for them inside the loop (where it would also wait
        // for the stage DMA in flight)
        __builtin_amdgcn_s_waitcnt(0);
#endif
        if (cur.x >= 0) {
            issue(cur.x, g * p.G + cur.hs, 0);
            const It d = n1.x >= 0 ? n1 : cur;   // (a copy nothing reads)
            n_flight = issue(d.x, g * p.G + d.hs, 1);
        }
        int buf = 0, par = 0;
        while (cur.x >= 0 || prv.x >= 0) {
            const It n2 = succ(n1);
            // this wave's DMA of stage t has landed (stage t + 1's may still be in
            // flight); after the barrier every wave's has, every wave is done with
            // the buffer the next request overwrites and with the exchange slot
            // the P waves write now
            switch (n_flight) {   // s_waitcnt vmcnt(n_flight) lgkmcnt(0) (operand must be a constant)
#if defined(__HIP_DEVICE_COMPILE__)
            case 0: __builtin_amdgcn_s_waitcnt(0x0070); break;
            case 2: __builtin_amdgcn_s_waitcnt(0x0072); break;
            case 3: __builtin_amdgcn_s_waitcnt(0x0073); break;
            case 4: __builtin_amdgcn_s_waitcnt(0x0074); break;
            case 5: __builtin_amdgcn_s_waitcnt(0x0075); break;
            case 6: __builtin_amdgcn_s_waitcnt(0x0076); break;
            case 7: __builtin_amdgcn_s_waitcnt(0x0077); break;
            default: __builtin_amdgcn_s_waitcnt(0x0070); break;
#endif
            }
            asm volatile("s_barrier" ::: "memory");
            {
                const It d = n2.x >= 0 ? n2 : (cur.x >= 0 ? cur : prv);   // (a copy nothing reads)
                n_flight = issue(d.x, g * p.G + d.hs, (buf + 2) & 3);     // stage t + 2
            }
            asm volatile("" ::: "memory");
            // the P wave's work is (block, head) t; the dS wave's is t - 1
            const It w = ROLE ? prv : cur;
            if (w.x >= 0) {
                const char* st = smem + (ROLE ? ((buf + 3) & 3) : buf) * STAGE;
                char* const xp = smem + XP_OFF + (ROLE ? par ^ 1 : par) * 8192 + kg * 2048 + 16 * lane;   // + 1024 h
                const int i0 = w.x * BM;
                const int hcur = g * p.G + w.hs;
                const int my_cls = (w.code >> (2 * xk)) & 3;
                const float* rsl = (const float*)(st + RS_OFF);

                // ---- S (P waves) or dP (dS waves): A operands are the Q or dO rows
                f32x16 sacc;
                {
                    const unsigned rows = lds_addr(st + (ROLE ? DO_OFF : Q_OFF));
                    bf16x8 ar[NKK];
                    unsigned aa[NKK];
#pragma unroll
                    for (int kk = 0; kk < NKK; ++kk)
                        aa[kk] = rows + (unsigned)(kl * (2 * D) + 16 * ((2 * kk + hh) ^ row_swz<D>(kl)));
                    lds_read16<NKK>(ar, aa);
                    sacc = f32x16{};
#pragma unroll
                    for (int kk = 0; kk < NKK; ++kk)
                        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ar[kk], kvreg[kk], sacc, 0, 0, 0);
                }

                bf16x8 pb[2];   // P (P waves) / dS (dS waves): queries 16 c + 8 (t / 4) + 4 hh + (t % 4)
                if (ROLE == 0) {
                    // ---- P = exp2(S c + bias log2(e) - lse2), masked
                    const int bc = bias_class(w.x);
                    const int* qil = (const int*)(st + QI_OFF);
                    const char* bsl = st + BS_OFF + kg * BSW + ES * (31 - kl);   // + slot * RUNB
                    auto body = [&](auto bct, auto mt) {
                        constexpr int BCT = decltype(bct)::value;
                        constexpr bool MASKED = decltype(mt)::value;
                        // (the stage's row statistics, query descriptors and bias runs, read
                        // in asm blocks: see lds_read16)
                        f32x4 rsv[8];
                        lds_read_pairs(rsv, lds_addr(rsl) + 32u * (unsigned)hh);
                        f32x4 qiv[8];
                        if constexpr (MASKED) lds_read_pairs(qiv, lds_addr(qil) + 32u * (unsigned)hh);
                        unsigned bvr[16];
                        if constexpr (BCT != BC_NONE) lds_read_bias<PB>(bvr, lds_addr(bsl) + (unsigned)(hh * RUNB));
                        // A run that starts before the block reads as 0 from a DMA piece at
                        // a wrapped offset: the block's first 8 entries are loaded here.  Only
                        // the rows of a block with i0 E < 8 can hold them (a uniform test);
                        // the loads are waited for inside the branch, so that no wait for
                        // them (which would also wait for the stage DMA) sits on other paths.
                        if constexpr (BCT == BC_EDGE) {
                            if (i0 * p.E < 8) {
                                const char* pr0 = (const char*)p.profiles + ((size_t)b * p.Hq + hcur) * pblock;
#pragma unroll
                                for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                                    for (int e = 0; e < 4; ++e) {
                                        const int m0 = 8 * jj + 4 * hh;
                                        const int r = p.qoff + i0 + m0 + e - j;
                                        const int ent = (i0 + m0 + e) * p.E + r;   // entry index in the block
                                        if (ent < 8 && (unsigned)r < (unsigned)p.E)
                                            bvr[4 * jj + e] = PB ? (unsigned)((const unsigned short*)pr0)[ent]
                                                                 : ((const unsigned*)pr0)[ent];
                                    }
#if defined(__HIP_DEVICE_COMPILE__)
                                __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
#endif
                            }
                        }
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            const int m0 = 8 * jj + 4 * hh;
                            const f32x4 rs01 = rsv[2 * jj];
                            const f32x4 rs23 = rsv[2 * jj + 1];
                            i32x4 qi01, qi23;
                            if constexpr (MASKED) {
                                qi01 = __builtin_bit_cast(i32x4, qiv[2 * jj]);
                                qi23 = __builtin_bit_cast(i32x4, qiv[2 * jj + 1]);
                            }
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float lse2 = e < 2 ? rs01[2 * e] : rs23[2 * (e - 2)];
                                float pre = -lse2;
                                if constexpr (BCT != BC_NONE) {
                                    float bias;
                                    if constexpr (PB)
                                        bias = __uint_as_float(bvr[4 * jj + e] << 16);
                                    else
                                        bias = __uint_as_float(bvr[4 * jj + e]);
                                    if constexpr (BCT == BC_FULL) pre = __builtin_fmaf(bias, LOG2E, -lse2);
                                    if constexpr (BCT == BC_EDGE) {
                                        const int r = p.qoff + i0 + m0 + e - j;
                                        pre = (unsigned)r < (unsigned)p.E ? __builtin_fmaf(bias, LOG2E, -lse2) : pre;
                                    }
                                }
                                float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[4 * jj + e], p.c_log2, pre));
                                if constexpr (MASKED) {
                                    const int gq = e < 2 ? qi01[2 * e] : qi23[2 * (e - 2)];
                                    const int aq = e < 2 ? qi01[2 * e + 1] : qi23[2 * (e - 2) + 1];
                                    pr = key_visible(gq, aq, j, c_k, wlim) ? pr : 0.0f;
                                }
                                pb[jj >> 1][4 * (jj & 1) + e] = (__bf16)pr;
                            }
                        }
                    };
                    using F = std::false_type;
                    using T = std::true_type;
                    using NONE = std::integral_constant<int, BC_NONE>;
                    using FULL = std::integral_constant<int, BC_FULL>;
                    using EDGE = std::integral_constant<int, BC_EDGE>;
                    if (my_cls == TILE_FULL) {
                        if (bc == BC_NONE) body(NONE{}, F{});
                        else if (bc == BC_FULL) body(FULL{}, F{});
                        else body(EDGE{}, F{});
                    } else {
                        if (bc == BC_NONE) body(NONE{}, T{});
                        else if (bc == BC_FULL) body(FULL{}, T{});
                        else body(EDGE{}, T{});
                    }
                    *(bf16x8*)(xp) = pb[0];
                    *(bf16x8*)(xp + 1024) = pb[1];
                } else {
                    // ---- dS = P (dP - (Delta - dlse)); dO (so dP) is 0 on rows that
                    // are not real or lie past Sq, and V on keys that are not real, so
                    // dP is finite everywhere and P = 0 masks dS
                    bf16x8 p0, p1;
                    lds_read_two(p0, p1, lds_addr(xp));
                    f32x4 rsv[8];
                    lds_read_pairs(rsv, lds_addr(rsl) + 32u * (unsigned)hh);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const f32x4 rs01 = rsv[2 * jj];
                        const f32x4 rs23 = rsv[2 * jj + 1];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float dlt = e < 2 ? rs01[2 * e + 1] : rs23[2 * (e - 2) + 1];
                            const int t = 4 * (jj & 1) + e;
                            const float pr = (float)((jj >> 1) ? p1[t] : p0[t]);
                            pb[jj >> 1][t] = (__bf16)(pr * (sacc[4 * jj + e] - dlt));
                        }
                    }
                }

                // ---- dV^T += dO^T P (P waves) or dK^T += Q^T dS (dS waves); the
                // transposed operands come from the rows by transposing LDS reads
                {
                    const unsigned rl = lds_addr(st + (ROLE ? Q_OFF : DO_OFF));
                    unsigned ad128[2 * NDB];   // D = 128: the reads of query step 0 (step 1 at + 4096)
                    if constexpr (D == 128) {
                        const unsigned x0 = rl + trb;
#pragma unroll
                        for (int db = 0; db < NDB; ++db) {
                            ad128[2 * db] = x0 ^ (64u * (unsigned)db);
                            ad128[2 * db + 1] = (x0 + 2048u) ^ (64u * (unsigned)db + 32u);
                        }
                    }
                    auto part = [&](auto cv) {
                        constexpr int c = decltype(cv)::value;
                        s16x4 rd[2 * NDB];
                        if constexpr (D == 128) {
                            tr_read<2 * NDB, 4096 * c>(rd, ad128);
                        } else {
                            unsigned ad[2 * NDB];
#pragma unroll
                            for (int db = 0; db < NDB; ++db) {
                                ad[2 * db] = rl + (unsigned)trof[c][0][db];
                                ad[2 * db + 1] = rl + (unsigned)trof[c][1][db];
                            }
                            tr_read<2 * NDB>(rd, ad);
                        }
#pragma unroll
                        for (int db = 0; db < NDB; ++db) {
                            const s16x4 lo = rd[2 * db], hi = rd[2 * db + 1];
                            const bf16x8 a =
                                __builtin_bit_cast(bf16x8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
                            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[c], acc[db], 0, 0, 0);
                        }
                    };
                    part(std::integral_constant<int, 0>{});
                    part(std::integral_constant<int, 1>{});
                }
            }
            asm volatile("" ::: "memory");
            buf = (buf + 1) & 3;
            par ^= 1;
            prv = cur;
            cur = n1;
            n1 = n2;
        }
    };
    if (role) kv_loop(std::integral_constant<int, 1>{});
    else kv_loop(std::integral_constant<int, 0>{});
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_s_waitcnt(0);   // no DMA outstanding at exit
#endif

    if (!kin) return;
    const size_t ko = (((size_t)b * p.Sk + j) * p.Hkv + g) * D;
    float* const dst = role ? p.dk : p.dv;
    const float sc = role ? p.scale : 1.0f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            f32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = acc[db][4 * jj + e] * sc;
            *(f32x4*)(dst + ko + 32 * db + 8 * jj + 4 * hh) = w;
        }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ x, size_t n)
{
    for (size_t u = (size_t)blockIdx.x * 256 + threadIdx.x; u < n; u += (size_t)gridDim.x * 256) x[u] = 0.0f;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
struct BwdLayout {
    size_t qinfo, rowstat, dob, total;
};

BwdLayout bwd_layout(int B, int Sq, int Sk, int Hq, int Hkv, int D)
{
    BwdLayout l;
    size_t o = summaries_bytes(B, Sq, Sk);
    l.qinfo = o;   o += round256((size_t)B * Sq * 8);
    l.rowstat = o; o += round256((size_t)B * Hq * Sq * 8);
    l.dob = o;     o += round256((size_t)B * Sq * Hq * D * 2);
    l.total = o;
    return l;
}

template <int D, bool PB>
int launch_bwd(const BwdParams& p, hipStream_t st)
{
    const long long rows = (long long)p.B * p.Sq * p.Hq;
    const int rpb = 256 / (D / 4);
    hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), 0, st, p);
    if (int rc = check_launch("bwd_prep_kernel")) return rc;
    const size_t ndq = (size_t)p.nQG * p.B * p.Hkv * p.nchunk;
    hipLaunchKernelGGL((bwd_dq_kernel<D, PB>), dim3((unsigned)ndq), dim3(64 * DQ_WAVES), 0, st, p);
    if (int rc = check_launch("bwd_dq_kernel")) return rc;
    const size_t nkv = (size_t)p.nKB * p.B * p.Hkv;
    if (nkv == 0) return INKATTN_OK;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, PB>), dim3((unsigned)nkv), dim3(64 * KV_WAVES), 0, st, p);
    return check_launch("bwd_dkdv_kernel");
}

}  // namespace

extern "C" {

size_t attn_bwd_workspace_size(int B, int Sq, int Sk, int Hq, int Hkv, int D)
{
    if (B <= 0 || Sq < 0 || Sk < 0 || Hq < 0 || Hkv < 0 || D < 0) return 0;
    return bwd_layout(B, Sq, Sk, Hq, Hkv, D).total;
}

int attn_bwd(const void* q, const void* k, const void* v, const void* profiles, int profiles_dtype,
             const float* sink, const uint8_t* valid, const uint8_t* key_valid, const int32_t* positions,
             const int32_t* key_positions, int64_t window, int64_t query_offset, int B, int Sq, int Sk, int Hq,
             int Hkv, int D, int E, const float* out, const float* lse, const float* dout, const float* dlse,
             float* dq, float* dk, float* dv, void* dprofiles, float* dsink, void* workspace,
             size_t workspace_bytes, void* stream)
{
    clear_error();
    if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
        return fail(INKATTN_ERR_SHAPE, "Hq=%d must be a positive multiple of Hkv=%d", Hq, Hkv);
    if (E < 1) return fail(INKATTN_ERR_SHAPE, "relative extent E=%d must be >= 1", E);
    if (D != 64 && D != 128) return fail(INKATTN_ERR_UNSUPPORTED, "head_dim %d not built (64, 128)", D);
    if (profiles_dtype != INKATTN_F32 && profiles_dtype != INKATTN_BF16)
        return fail(INKATTN_ERR_UNSUPPORTED, "profiles dtype %d unknown", profiles_dtype);
    MaskArgs ma;
    if (int rc = resolve_mask_args(valid, key_valid, positions, key_positions, query_offset, B, Sq, Sk, &ma))
        return rc;
    if ((size_t)B * Sq * Hq * D >= (size_t(1) << 40) || (size_t)B * Hq * Sq * E >= (size_t(1) << 40))
        return fail(INKATTN_ERR_SHAPE, "tensor too large");
    if ((size_t)Sq * E * (profiles_dtype == INKATTN_F32 ? 4 : 2) >= (size_t(1) << 32) - (size_t(1) << 20))
        return fail(INKATTN_ERR_SHAPE, "one (batch row, head) block of profiles must stay below 4 GiB - 1 MiB");
    if ((size_t)Sk * Hkv * D * 2 >= (size_t(1) << 32) || (size_t)Sq * Hq * D * 2 >= (size_t(1) << 32))
        return fail(INKATTN_ERR_SHAPE, "one batch row of q, k or v must stay below 4 GiB");
    const int nQB = ceil_div(Sq, BM), nKT = ceil_div(Sk, BN);
    if ((size_t)B * Hq * nQB >= (size_t(1) << 31) || (size_t)B * Hkv * nKT >= (size_t(1) << 31))
        return fail(INKATTN_ERR_SHAPE, "too many tiles");
    if ((size_t)B * Sq == 0 && (size_t)B * Sk == 0) return INKATTN_OK;
    hipStream_t st = (hipStream_t)stream;
    if ((size_t)B * Sq == 0) {   // no query: every key gradient is 0 (no other tensor is read)
        if (!dk || !dv) return fail(INKATTN_ERR_NULL, "dk or dv is NULL");
        if (!aligned(dk, 16) || !aligned(dv, 16)) return fail(INKATTN_ERR_ALIGN, "dk and dv must be 16-byte aligned");
        const size_t n = (size_t)B * Sk * Hkv * D;
        const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 65536);
        hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, st, dk, n);
        hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, st, dv, n);
        return check_launch("fill_zero_kernel");
    }
    if (!q || !profiles || !sink || !out || !lse || !dout || !dq || !dprofiles || !dsink)
        return fail(INKATTN_ERR_NULL, "q/profiles/sink/out/lse/dout/dq/dprofiles/dsink is NULL");
    if (Sk > 0 && (!k || !v || !dk || !dv)) return fail(INKATTN_ERR_NULL, "k, v, dk or dv is NULL");
    if (!aligned(q, 16) || !aligned(out, 16) || !aligned(dout, 16) || !aligned(dq, 16) ||
        (Sk > 0 && (!aligned(k, 16) || !aligned(v, 16) || !aligned(dk, 16) || !aligned(dv, 16))))
        return fail(INKATTN_ERR_ALIGN, "q, k, v, out, dout, dq, dk and dv must be 16-byte aligned");
    const size_t pal = profiles_dtype == INKATTN_F32 ? 4 : 2;
    if (!aligned(profiles, pal) || !aligned(dprofiles, pal) || !aligned(sink, 4) || !aligned(lse, 4) ||
        !aligned(dsink, 4) || (dlse && !aligned(dlse, 4)))
        return fail(INKATTN_ERR_ALIGN, "profiles / dprofiles / sink / lse / dlse / dsink misaligned");
    const BwdLayout lay = bwd_layout(B, Sq, Sk, Hq, Hkv, D);
    if (int rc = check_workspace(workspace, workspace_bytes, lay.total)) return rc;
    const int w = (window <= 0 || window >= (int64_t(1) << 31)) ? 0 : (int)window;
    if (int rc = launch_summaries(valid, positions, ma.key_valid, ma.key_positions, (int)query_offset, B, Sq, Sk,
                                  workspace, st))
        return rc;

    char* ws = (char*)workspace;
    BwdParams p;
    p.q = (const __bf16*)q;
    p.k = (const __bf16*)k;
    p.v = (const __bf16*)v;
    p.profiles = profiles;
    p.sink = sink;
    p.out = out;
    p.lse = lse;
    p.dout = dout;
    p.dlse = dlse;
    p.valid = valid;
    p.key_valid = ma.key_valid;
    p.positions = positions;
    p.qsum = (const TileSummary*)ws;
    p.ksum = p.qsum + (size_t)B * nQB;
    p.kanchor = (const int*)(ws + tile_summary_bytes(B, Sq, Sk));
    p.qinfo = (int2*)(ws + lay.qinfo);
    p.rowstat = (float2*)(ws + lay.rowstat);
    p.dob = (__bf16*)(ws + lay.dob);
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.dprofiles = dprofiles;
    p.dsink = dsink;
    p.B = B; p.Sq = Sq; p.Sk = Sk; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv; p.E = E;
    p.window = w;
    p.qoff = (int)query_offset;
    p.hpw = (p.G % 4 == 0) ? 4 : (p.G % 2 == 0) ? 2 : 1;
    p.tpw = BW_WAVES / p.hpw;
    p.nchunk = p.G / p.hpw;
    p.nQB = nQB;
    p.nKT = nKT;
    p.nQG = ceil_div(nQB, p.tpw);
    p.nKB = ceil_div(Sk, KV_KEYS);
    p.scale = 1.0f / sqrtf((float)D);
    p.c_log2 = p.scale * LOG2E;
    if ((size_t)p.nQG * B * Hkv * p.nchunk >= (size_t(1) << 31)) return fail(INKATTN_ERR_SHAPE, "grid too large");
    const bool pb = profiles_dtype == INKATTN_BF16;
    if (D == 128) return pb ? launch_bwd<128, true>(p, st) : launch_bwd<128, false>(p, st);
    return pb ? launch_bwd<64, true>(p, st) : launch_bwd<64, false>(p, st);
}

}  // extern "C"
