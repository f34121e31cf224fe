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
//   1. summarize_kernel (scheduler pre-pass, one wave per tile): for every
//      32-token query block and 64-key tile, the min / max document start
//      column over real tokens and the number of real tokens, plus each key's
//      start column.  Every skip / full / masked decision of the main kernel
//      comes from these summaries.
//   2. stage_values_kernel: v (bf16) -> fp16 V^T per 64-key tile, keys in the
//      order the PV product consumes them, zero at keys that are not real
//      (the probabilities multiply the values in fp16).
//   3. attn_fwd_kernel: one workgroup per (batch row, K/V head, head chunk,
//      group of 32-token query blocks); each wave owns one (query head,
//      32-token block).  Each 64-key K / V^T tile is staged once in LDS by DMA
//      (buffer_load ... lds, XOR-swizzled rows) and serves every wave of the
//      workgroup, i.e. every query head of the chunk (GQA).  The next live
//      tile's DMA is issued at the start of the current tile, this wave's
//      bias for it after the current tile's S^T (one barrier per tile).
//      Tiles on which no wave of the workgroup can take bias run a loop body
//      without the bias code.  Per wave and tile:
//        S^T = K Q^T      bf16 MFMA 32x32x16 as two interleaved chains (one per
//                         32-key half), keys on M and queries on N, so each
//                         lane owns one query column: row reductions are
//                         in-lane plus one exchange between the wave halves;
//        + bias           the relative bias times sqrt(D), from the query's
//                         own profile row, staged one tile ahead in a per-wave
//                         LDS strip by DMA (whole row strips, 4-entry runs or
//                         single entries, by how the tile meets [0, E));
//        mask             only on tiles classed as masked;
//        online softmax   a running frame and denominator per lane over the
//                         64 keys, started from the sink logit (the sink's
//                         weight enters the denominator, never the value
//                         sum); no per-tile row max: the frame moves (to the
//                         row max, with an output rescale) only when a
//                         lane's sum of its fp16 weights reaches 2^15, which
//                         keeps every weight inside fp16's range;
//        O^T += V^T P^T   fp16 MFMA 32x32x16; P^T comes straight from the S^T
//                         accumulator registers and V^T is one 16-byte LDS
//                         read per lane and MFMA (the staging pass put the
//                         keys in the same order as P^T's).
//      Epilogue: out = O / l, lse = ln(2) * (m + log2 l).
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "common.h"
#include "inkattn.h"

namespace {

using namespace inkattn;

constexpr int NWAVES = 8; // waves per attention workgroup (one workgroup per CU)
constexpr float FRAME_LIMIT = 32768.0f;   // bound on a lane's partial sum of 32 fp16 weights in the frame
// s_waitcnt operands (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8):
// vmcnt(0) lgkmcnt(0); lgkmcnt(0) alone
[[maybe_unused]] constexpr int WAIT_VM_LGKM = 0x0070;   // (used by the device pass only)
[[maybe_unused]] constexpr int WAIT_LGKM = 0xC07F;



// ---------------------------------------------------------------------------
// Scheduler pre-pass: one wave per (batch row, tile); query tiles first, then
// key tiles, in one launch.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int wave_min(int x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ __forceinline__ int wave_max(int x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o, 64));
    return x;
}

__global__ __launch_bounds__(256) void summarize_kernel(
    const uint8_t* __restrict__ valid, const int32_t* __restrict__ positions, int qoff, int Sq, int nQB,
    const uint8_t* __restrict__ key_valid, const int32_t* __restrict__ key_positions, int Sk, int nKT,
    int B, TileSummary* __restrict__ qsum, TileSummary* __restrict__ ksum, int* __restrict__ kanchor)
{
    const int w = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int nq = B * nQB;
    if (w >= nq + B * nKT) return;   // whole wave exits together
    const bool is_q = w < nq;
    const int t = is_q ? w : w - nq;
    const int ntiles = is_q ? nQB : nKT;
    const int b = t / ntiles, tile = t - b * ntiles;
    const int size = is_q ? BM : BN;
    const int S = is_q ? Sq : Sk;
    const uint8_t* vld = is_q ? valid : key_valid;
    const int32_t* pos = is_q ? positions : key_positions;
    const int col0 = is_q ? qoff : 0;
    const int i = tile * size + lane;
    int amin = INT_MAX, amax = INT_MIN, n = 0;
    if (lane < size && i < S) {
        const size_t o = (size_t)b * S + i;
        if (vld[o]) {
            const int a = pos ? col0 + i - pos[o] : 0;
            amin = a; amax = a; n = 1;
        }
    }
    // per-key start column for the masked tiles, INT_MIN for keys that are not
    // real and for the padding of the last tile
    if (!is_q) kanchor[(size_t)b * ntiles * BN + i] = n ? amin : INT_MIN;
    amin = wave_min(amin);
    amax = wave_max(amax);
    n = __popcll(__builtin_amdgcn_ballot_w64(n != 0));
    if (lane == 0) {
        TileSummary s;
        s.amin = amin; s.amax = amax; s.nvalid = n; s.pad = 0;
        (is_q ? qsum : ksum)[t] = s;
    }
}

struct FwdParams {
    const __bf16* q;
    const __bf16* k;
    const _Float16* v16;           // values converted to fp16 (zero at keys that are not real)
    const void* profiles;
    const float* sink;
    const uint8_t* valid;
    const uint8_t* key_valid;
    const int32_t* positions;      // NULL: global column
    const int32_t* key_positions;  // NULL: key column
    const TileSummary* qsum;       // [B, nQB]
    const TileSummary* ksum;       // [B, nKT]
    const int* kanchor;            // [B, Sk] key start column j - key_positions[j], INT_MIN if not real
    const __bf16* rfeat;           // relative features [.., d_rel] (profiles formed in-kernel), or NULL
    const __bf16* table;           // relative table rows [E, d_rel] of this launch's heads
    long long r_bs, r_ts, r_hs;    // element strides (batch row, token, head) of rfeat
    long long t_hs;                // elements between the table slices of two heads (0: one shared slice)
    void* out;                     // fp32, or bf16 when out_bf16
    float* lse;                    // may be NULL (not written)
    // element strides (batch row, token, head) of q, k, out, lse and sink
    long long q_bs, q_ts, q_hs, k_bs, k_ts, k_hs, o_bs, o_ts, o_hs, l_bs, l_ts, l_hs, s_bs, s_ts, s_hs;
    int out_bf16;
    int B, Sq, Sk, Hq, Hkv, G, E;  // E == 0: no relative bias (profiles unused)
    int window;      // <= 0: none
    int qoff;        // query_offset
    int hpw;         // query heads per workgroup
    int tpw;         // 32-token query blocks per workgroup (hpw * tpw == waves)
    int nchunk;      // head chunks per K/V head (G / hpw)
    int nQB, nQG, nKT;
    float c_log2;    // head_dim^-0.5 * log2(e)
};


// Wait for every outstanding memory operation of the wave, then meet the
// workgroup.  The wait is the builtin so that the compiler's own wait counting
// knows of it; the barrier is an asm statement with a memory clobber so that
// no memory access moves across it.
__device__ __forceinline__ void wait_all_and_barrier()
{
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_s_waitcnt(WAIT_VM_LGKM);
#endif
    asm volatile("s_barrier" ::: "memory");
}

// As wait_all_and_barrier, but the last n_after vector-memory loads of the
// wave (n_after in {0, 4, 5, 8, 16, 20, 32}) may still be in flight.  s_waitcnt
// operand: vmcnt in bits 3:0 and 15:14, expcnt 6:4 (7: no wait), lgkmcnt 11:8.
__device__ __forceinline__ void wait_dma_and_barrier(int n_after)
{
#if defined(__HIP_DEVICE_COMPILE__)
    switch (n_after) {
    case 4: __builtin_amdgcn_s_waitcnt(0x0074); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0075); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0078); break;
    case 16: __builtin_amdgcn_s_waitcnt(0x4070); break;
    case 20: __builtin_amdgcn_s_waitcnt(0x4074); break;
    case 32: __builtin_amdgcn_s_waitcnt(0x8070); break;
    default: __builtin_amdgcn_s_waitcnt(WAIT_VM_LGKM); break;
    }
#endif
    asm volatile("s_barrier" ::: "memory");
}

// Waits until at most n (3 or 5) vector-memory instructions of the wave are outstanding.
__device__ __forceinline__ void wait_vm_keep(int n)
{
#if defined(__HIP_DEVICE_COMPILE__)
    if (n == 3) __builtin_amdgcn_s_waitcnt(0x0F73);
    else if (n == 5) __builtin_amdgcn_s_waitcnt(0x0F75);
    else __builtin_amdgcn_s_waitcnt(0x0F70);
#endif
}

// Max / sum of a value and its twin in the other wave half (same query).
__device__ __forceinline__ float half_max(float x)
{
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float half_sum(float x)
{
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Tile descriptor carried through the software pipeline.
struct TileDesc {
    int kt;        // tile index (> kt_hi: none)
    int my_cls;    // this wave's class
};

// LDS layout of one staged K tile.  Each 16-byte DMA instruction writes
// 1 KB of LDS contiguously, i.e. RPI whole rows, so rows cannot be padded
// one by one; instead rows come in groups of RPI (pitch KGP bytes) and the
// 16-byte chunks of a row are XOR-swizzled, which makes the MFMA operand
// reads (16 rows x 16 B per phase) bank-conflict free on the 64-bank LDS.
template <int D> struct TileLayout;
template <> struct TileLayout<128> {
    static constexpr int RPI = 4, KGP = 1088;
    __device__ static constexpr int ksw(int t) { return t; }
};
template <> struct TileLayout<64> {
    static constexpr int RPI = 8, KGP = 1088;
    __device__ static constexpr int ksw(int t) { return t >> 1; }
};


// REL > 0: the profile rows are not read but formed in-kernel from REL
// relative features per (token, head) and the relative table (see the bias
// section); REL == 0: the profiles tensor is read.
template <int D, bool PROF_BF16, int NW, int REL>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(FwdParams p)
{
    using L = TileLayout<D>;
    constexpr int NKK = D / 16;              // k-steps of S^T = K Q^T
    constexpr int NDB = D / 32;              // 32-row d-blocks of O^T
    constexpr int CPR = D / 8;               // 16-byte chunks per row
    constexpr int NGRP = BN / L::RPI;        // DMA groups per tile (per tensor)
    constexpr int GPW = NGRP / NW;           // DMA groups per wave
    static_assert(NGRP % NW == 0, "DMA groups must divide among waves");
    constexpr int KBYTES = NGRP * L::KGP;
    constexpr int VBYTES = D * 128;          // one V^T tile: D rows of 64 fp16
    constexpr int NVG = D / 8;               // 1 KB DMA groups per V^T tile (8 rows each)
    static_assert(NVG % NW == 0 && NW % 2 == 0, "V^T DMA groups must divide among an even number of waves");
    // K and the start columns double-buffered; V triple-buffered (the PV
    // product of a tile runs during the next tile, while the tile after that
    // is being fetched)
    constexpr int K_OFF = 0, V_OFF = 2 * KBYTES, CA_OFF = 2 * KBYTES + 3 * VBYTES;
    // fp32 bias strips: per wave 32 rows x 64 distances (8 KB), staged by
    // DMA; formed in-kernel (REL > 0) they take rows of 272 bytes (64
    // distances + 16 bytes of padding, which spreads the rows over the banks)
    static_assert(REL == 0 || REL == 16 || REL == 32, "relative feature widths 16 and 32 are built");
    constexpr int SROW = REL ? 272 : BN * 4;
    constexpr int BSTRIP = BM * SROW;
    constexpr int B_OFF = CA_OFF + 2 * BN * 4;
    // tile schedule: one entry per live key tile of a round of NSCHED tiles,
    // plus a count per wave
    constexpr int NSCHED = 64 * NW;
    constexpr int SCHED_OFF = B_OFF + NW * BSTRIP;
    constexpr int LDS_BYTES = SCHED_OFF + (NSCHED + NW) * 4;
    // vector-memory instructions of one tile's K / V / start-column DMA (per wave)
    constexpr int N_KV_DMA = NGRP / NW + NVG / NW + 1;

    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qi = lane & 31;      // this lane's query within the block
    const int hh = lane >> 5;      // wave half

    // ---- work item: head groups fastest, then batch rows, then query groups in
    // decreasing order (longest first for causal work).
    int idx = blockIdx.x;
    const int ngroups = p.Hkv * p.nchunk;
    // (divisions by kernel arguments go through the vector unit: readfirstlane
    // tells the compiler that these wave-uniform values are, so the buffer
    // resources built from them stay in scalar registers)
    const int hgi = __builtin_amdgcn_readfirstlane(idx % ngroups); idx /= ngroups;
    const int b = __builtin_amdgcn_readfirstlane(idx % p.B); idx /= p.B;
    const int qg = __builtin_amdgcn_readfirstlane(p.nQG - 1 - idx);
    const int g = __builtin_amdgcn_readfirstlane(hgi / p.nchunk);
    const int h = __builtin_amdgcn_readfirstlane(g * p.G + (hgi - g * p.nchunk) * p.hpw + wave % p.hpw);
    const int qb = __builtin_amdgcn_readfirstlane(qg * p.tpw + wave / p.hpw);   // this wave's query block (may be past the end)
    const int i0 = qb * BM;

    // query blocks of the workgroup: qg*tpw .. qg*tpw + tpw - 1
    const int qb_first = qg * p.tpw;
    const int qb_last = min(p.nQB - 1, qb_first + p.tpw - 1);

    const int i = i0 + qi;
    const bool qin = qb < p.nQB && i < p.Sq;
    const size_t qrow = (size_t)b * p.Sq + i;
    const int gi = p.qoff + i;
    const bool qreal = qin && p.valid[qrow] != 0;
    const int a_q = qreal ? (p.positions ? gi - p.positions[qrow] : 0) : 0;
    const int gi_eff = qreal ? gi : -1;
    const unsigned wlim = p.window > 0 ? (unsigned)p.window : 0x80000000u;
    const float sig = (qin && p.sink) ? p.sink[b * p.s_bs + i * p.s_ts + h * p.s_hs] : -INFINITY;

    // Q^T operand: lane holds q[i, h, 16*kk + 8*hh + 0..7].
    bf16x8 qreg[NKK];
    {
        const __bf16* qp = p.q + b * p.q_bs + (long long)i * p.q_ts + h * p.q_hs + 8 * hh;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) qreg[kk] = qin ? *(const bf16x8*)(qp + 16 * kk) : bf16x8{};
    }
    // relative features (REL > 0), the B operand of the profile product:
    // lane holds rfeat[i, h, 16*kk + 8*hh + 0..7]
    constexpr int NRK = REL ? REL / 16 : 1;
    bf16x8 rreg[NRK];
#pragma unroll
    for (int kk = 0; kk < NRK; ++kk) rreg[kk] = bf16x8{};
    if constexpr (REL > 0) {
        const __bf16* rp = p.rfeat + b * p.r_bs + (long long)i * p.r_ts + h * p.r_hs + 8 * hh;
#pragma unroll
        for (int kk = 0; kk < NRK; ++kk) rreg[kk] = qin ? *(const bf16x8*)(rp + 16 * kk) : bf16x8{};
    }

    // Online-softmax state (log2 units).  The sink's weight e^{s - m} counts
    // once, in the lower half's partial denominator.
    float m = sig * LOG2E;              // -inf when there is no sink
    float l = (hh == 0 && sig != -INFINITY) ? 1.0f : 0.0f;
    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};

    // ---- this wave's block and the workgroup's key-tile range
    int qcount = 0;
    if (qb < p.nQB) qcount = min(BM, p.Sq - i0);
    const int qlo = p.qoff + i0, qhi = p.qoff + i0 + qcount - 1;

    int jlo = INT_MAX, jhi = -1;
    for (int x = qb_first; x <= qb_last; ++x) {
        const TileSummary s = p.qsum[(size_t)b * p.nQB + x];
        if (s.nvalid == 0) continue;
        const int xlo = p.qoff + x * BM;
        const int xhi = p.qoff + min(p.Sq, x * BM + BM) - 1;
        int lo = max(0, s.amin);                         // key j >= its start column
        if (p.window > 0) lo = max(lo, xlo - p.window + 1);
        jlo = min(jlo, lo);
        jhi = max(jhi, min(p.Sk - 1, xhi));
    }
    const int kt_lo = jhi >= 0 ? jlo / BN : 0;
    const int kt_hi = jhi >= 0 ? jhi / BN : -1;

    // ---- tile schedule.  A round classifies key tiles base .. base + NSCHED - 1
    // (one per thread) against every query block of the workgroup and lists
    // the live ones in LDS in order: entry = (kt - base) | the class of query
    // block qb_first + x in bits 16 + 2 x .. 17 + 2 x.  Rounds are built by the
    // whole workgroup between barriers.
    int* sched = (int*)(smem + SCHED_OFF);
    auto build_round = [&](int base) -> int {
        const int kt = base + tid;
        unsigned code = 0;
        bool live = false;
        if (kt <= kt_hi) {
            const int j0 = kt * BN;
            const int kcount = min(BN, p.Sk - j0);
            const TileSummary ks = p.ksum[(size_t)b * p.nKT + kt];
            for (int x = qb_first; x <= qb_last; ++x) {
                const TileSummary qs = p.qsum[(size_t)b * p.nQB + x];
                const int xc = min(BM, p.Sq - x * BM);
                const int xlo = p.qoff + x * BM;
                const int c = classify_tile(qs, xlo, xlo + xc - 1, xc, ks, j0, j0 + kcount - 1, kcount, p.window);
                code |= (unsigned)c << (16 + 2 * (x - qb_first));
                live |= c != TILE_SKIP;
            }
        }
        const unsigned long long bal = __builtin_amdgcn_ballot_w64(live);
        const int before = __popcll(bal & ((1ull << lane) - 1ull));
        wait_all_and_barrier();                 // the previous round's entries are read
        if (lane == 0) sched[NSCHED + wave] = __popcll(bal);
        wait_all_and_barrier();
        int off = 0, total = 0;
        for (int w = 0; w < NW; ++w) {
            const int cw = sched[NSCHED + w];
            off += w < wave ? cw : 0;
            total += cw;
        }
        if (live) sched[off + before] = (int)(code | (unsigned)(kt - base));
        wait_all_and_barrier();
        return __builtin_amdgcn_readfirstlane(total);
    };
    int round_base = kt_lo, round_n = 0, round_i = 0;
    // Next live tile (some wave of the workgroup needs it), in order; uniform.
    auto next_live = [&]() -> TileDesc {
        while (round_i >= round_n && round_base <= kt_hi) {
            round_n = build_round(round_base);
            round_base += NSCHED;
            round_i = 0;
        }
        TileDesc d;
        if (round_i < round_n) {
            const unsigned w = (unsigned)__builtin_amdgcn_readfirstlane(sched[round_i]);
            d.kt = round_base - NSCHED + (int)(w & 0xFFFFu);
            d.my_cls = (int)((w >> (16 + 2 * (qb - qb_first))) & 3u);
            ++round_i;
        } else {
            d.kt = kt_hi + 1;
            d.my_cls = TILE_SKIP;
        }
        return d;
    };

    // ---- K / V staging by LDS DMA.  The K resource covers rows 0..Sk-1 of
    // this (batch row, K/V head), rows past Sk read as zero (their offsets
    // lie past the resource's size); the V^T resource covers the staged tiles
    // of this (batch row, K/V head).
    const int krow = (int)p.k_ts * 2;                   // bytes between consecutive keys
    const unsigned nrec = p.Sk > 0 ? (unsigned)((size_t)(p.Sk - 1) * krow + D * 2) : 0u;
    const __amdgpu_buffer_rsrc_t krsrc = uniform_rsrc(p.k + b * p.k_bs + g * p.k_hs, nrec);
    const __amdgpu_buffer_rsrc_t vrsrc = uniform_rsrc(
        p.v16 + ((size_t)b * p.Hkv + g) * p.nKT * (size_t)(D * BN), (size_t)p.nKT * VBYTES);
    // K: lane -> (row t of its DMA group, LDS chunk slot pc): it fetches the chunk that lands there
    const int dt = lane / CPR, dpc = lane % CPR;
    const int kvoff = dt * krow + 16 * (dpc ^ L::ksw(dt));
    // V^T: lane -> (row 8 a + lane / 8 of DMA group a, LDS chunk lane % 8); the
    // groups of a wave all have the parity of the wave (NW is even)
    const int vvoff = (lane / 8) * 128 + 16 * ((lane % 8) ^ vt_swz(8 * (wave & 1) + lane / 8));
    // key start columns of this batch row, padded to whole tiles with INT_MIN
    const __amdgpu_buffer_rsrc_t arsrc = uniform_rsrc(p.kanchor + (size_t)b * p.nKT * BN, (size_t)p.nKT * BN * 4);
    auto issue_tile = [&](const TileDesc& d, int bufsel, int vsel) {
        const int j0 = d.kt * BN;
#pragma unroll
        for (int u = 0; u < GPW; ++u) {
            const int a = wave + NW * u;                   // DMA group (uniform)
            // (the offsets are named values: an expression written into the
            // builtin's argument list keeps the host pass from emitting the
            // kernel's launch stub)
            // the whole byte offset travels in the offset register, which the
            // buffer range check covers: rows past Sk read as zero
            const int voff = kvoff + (j0 + a * L::RPI) * krow;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                krsrc, (lds_void*)(smem + K_OFF + bufsel * KBYTES + a * L::KGP), 16, voff, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < NVG / NW; ++u) {
            const int a = wave + NW * u;
            const int soff = d.kt * VBYTES + a * 1024;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                vrsrc, (lds_void*)(smem + V_OFF + vsel * VBYTES + a * 1024), 16, vvoff, soff, 0, 0);
        }
        // the tile's 64 key start columns, one dword per lane; every wave
        // writes the same values, so that each wave's sequence of memory
        // instructions is the same on every path (the compiler then counts
        // the outstanding ones exactly)
        const int asoff = j0 * 4;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            arsrc, (lds_void*)(smem + CA_OFF + bufsel * BN * 4), 4, 4 * lane, asoff, 0, 0);
    };

    // Per-lane LDS byte offsets of the MFMA operands within one buffer.  The
    // K swizzle XORs at most the two low bits of the chunk index, so the
    // chunk of k-step kk sits at 32*kk from one of two lane bases (even / odd kk).
    // Accumulator element (jj, e) of a 32-key half is key 8 jj + 4 hh + (e ^ 3): the
    // K row a lane supplies is qi ^ 3, so that keys 4k..4k+3 appear in
    // decreasing order, the order of increasing distance, i.e. the memory
    // order of a profile run.
    const int krow_lane = qi ^ 3;
    const int kt_row = krow_lane % L::RPI;
    const int ksw = L::ksw(kt_row);
    const int krowbase = (krow_lane / L::RPI) * L::KGP + kt_row * (2 * D) + 16 * (hh ^ (ksw & 1));
    const int kbase_even = krowbase + 32 * (ksw >> 1);
    const int kbase_odd = krowbase - 32 * (ksw >> 1);
    // V^T operand of 16-key step c: row qi (+ 32 per d-block), chunk 2 c + hh
    // (offsets in phase_pv)

    // ---- relative bias.  Element (jj, e) of half s of a tile's S^T
    // accumulator is key j0 + 32 s + 8 jj + 4 hh + (e ^ 3), i.e. distance
    // R - 32 s - 8 jj - 4 hh - (e ^ 3) with R = gi - j0.  All loads go through
    // a buffer resource over this (batch row, head)'s [Sq, E] block; the
    // hardware range-checks each offset register as an unsigned value, so
    // offsets past the block, or before it (wrapped), read as 0.
    constexpr int PE = PROF_BF16 ? 2 : 4;               // bytes per profile entry
    const __amdgpu_buffer_rsrc_t prsrc = uniform_rsrc(
        (const char*)p.profiles + ((size_t)b * p.Hq + h) * p.Sq * p.E * PE, (size_t)p.Sq * p.E * PE);
    constexpr float INV_SCALE = D == 128 ? 11.313708498984761f : 8.0f;   // sqrt(D)

    // Every bias value reaches the accumulators through this wave's 8 KB LDS
    // strip, filled by DMA one tile ahead, in one layout: row r (query
    // i0 + r) at bytes 256 r holds the distances R_r - 63 .. R_r of the tile
    // (R_r = its R), 4 bytes per distance, the 16-byte chunk c (distances
    // R_r - 63 + 4 c .. + 3) at slot c ^ (r % 16), which makes the reads of
    // the S^T layout conflict free.  Distances below 0 read whatever the
    // profile row before holds (finite; those keys are masked: they lie after
    // the query); distances >= E are zeroed on reading (BC_FAR).  Two ways in:
    //  - BC_ROWS (fp32): 16-byte runs, 4 rows per instruction, 8 instructions;
    //    only when the tile's lowest offset (row 0, distance R_0 - 63) lies
    //    inside the block, so that no run straddles its start;
    //  - BC_ENTRIES (fp32 near the block's start): one instruction per row,
    //    each lane one entry at its exact offset (64 contiguous entries per
    //    instruction).
    // bf16 profiles keep 2 bytes per entry: row r at 144 r holds a window of
    // 72 entries starting at the 4-byte boundary at or before the row's first
    // needed entry (clamped at the block start), as 9 dword-aligned 16-byte
    // runs, 5 instructions per tile (BC_ROWS); the reads shift each entry
    // group out of three dwords.
    enum : int { BC_NONE = 0, BC_ROWS = 1, BC_ENTRIES = 2, BC_FAR = 4 };
    char* bstrip = smem + B_OFF + wave * BSTRIP;

    // Issues the bias loads of this wave's part of tile d; returns its code.
    auto load_bias = [&](const TileDesc& d) -> int {
        if (p.E <= 0 || d.kt > kt_hi || d.my_cls == TILE_SKIP) return BC_NONE;
        const int j0n = d.kt * BN;
        if (qlo - (j0n + BN - 1) >= p.E) return BC_NONE;        // every distance >= E
        const int far = (qhi - j0n >= p.E) ? BC_FAR : 0;
        const int min_off = i0 * p.E + qlo - j0n - (BN - 1);    // entry of row 0, distance R_0 - 63
        __builtin_amdgcn_s_waitcnt(WAIT_LGKM);   // earlier reads of the strip are done
        lds_char* const bs = opaque_lds((lds_char*)bstrip);
        const unsigned ln = opaque((unsigned)lane);   // offsets derived per tile, not held in registers
        if constexpr (PROF_BF16) {
            // bf16: row r's window of 72 entries from a0 = max(s0 & ~1, 0) (s0 = min_off + r (E + 1),
            // its first needed entry), 9 dword-aligned 16-byte runs at 144 r + 16 c of the strip;
            // instruction u, lane L takes run g = 64 u + L (r = g / 9, c = g % 9), 288 runs in 5
            // instructions, the 32 lanes past them reading nothing (offsets out of range)
            const unsigned e1 = opaque_s((unsigned)(p.E + 1));
#pragma unroll
            for (int u = 0; u < 5; ++u) {
                const unsigned g = 64u * (unsigned)u + ln;
                const unsigned r = (g * 57u) >> 9;                  // g / 9 for g < 320
                const unsigned c = g - 9u * r;
                const int s0 = min_off + (int)(r * e1);
                const unsigned a0 = (unsigned)max(s0 & ~1, 0);
                const unsigned off = opaque(g < 288u ? (a0 + 8u * c) * 2u : 0xFFFFFFF0u);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(prsrc, (lds_void*)(bs + 1024 * u), 16, off, 0, 0, 0);
            }
            return BC_ROWS | far;
        }
        if (min_off >= 0) {
            // row r = 4 u + lane / 16 takes chunk (lane % 16) ^ (r % 16) = ((lane % 16) ^ (lane / 16)) ^ 4 (u % 4)
            const unsigned bl = (ln >> 4) * (unsigned)(p.E + 1) * 4u;
            const unsigned rstep = opaque_s((unsigned)(p.E + 1) * 16u);   // bytes between rows 4 apart, + 16
            const unsigned xb = 16u * ((ln & 15u) ^ (ln >> 4));
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const unsigned voff = opaque((unsigned)min_off * 4u + (unsigned)u * rstep + bl +
                                             (xb ^ (64u * (unsigned)(u & 3))));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(prsrc, (lds_void*)(bs + 1024 * u), 16, voff, 0, 0, 0);
            }
            return BC_ROWS | far;
        }
        // row r: lane L fetches distance R_r - 63 + (L ^ 4 (r % 16)), the entry its slot holds
        const unsigned rstep = opaque_s((unsigned)(p.E + 1));
#pragma unroll
        for (int r = 0; r < BM; ++r) {
            const unsigned off = opaque(((unsigned)min_off + (unsigned)r * rstep + (ln ^ (4u * (unsigned)(r & 15)))) *
                                        (unsigned)PE);
            if constexpr (PROF_BF16)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(prsrc, (lds_void*)(bs + 256 * r), 2, off, 0, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(prsrc, (lds_void*)(bs + 256 * r), 4, off, 0, 0, 0);
        }
        return BC_ENTRIES | far;
    };
    // Vector-memory instructions load_bias issued for a code.
    auto bias_loads = [&](int code) -> int {
        return (code & BC_ROWS) ? (PROF_BF16 ? 5 : 8) : (code & BC_ENTRIES) ? BM : 0;
    };
    // Adds tile j0t's bias (code as load_bias returned it) times sqrt(D) to the
    // accumulators.  Its loads were issued before this wave's DMA of the next
    // K / V tile, which may stay outstanding (N_KV_DMA instructions).
    auto bias_add_tile = [&](int code, int j0t, f32x16* a) {
        if (code == BC_NONE) return;
        wait_vm_keep(N_KV_DMA);
        const unsigned ln = opaque((unsigned)lane);   // offsets derived per tile, not held in registers
        f32x4 w[2][4];
        if constexpr (PROF_BF16) {
            // row qi's window starts delta entries before its first needed entry s0 (delta 0 or 1,
            // negative where the window was clamped at the block start: the entries before it are
            // those of keys after the query, masked); chunk k's 4 entries start at window entry
            // delta + 4 k, i.e. byte 2 (delta & 1) of dword (delta >> 1) + 2 k, and are shifted
            // out of three dwords (bf16 -> fp32: the entry is the upper half)
            const int s0 = i0 * p.E + qlo - j0t - (BN - 1) + (int)(ln & 31u) * (p.E + 1);
            const int delta = s0 - max(s0 & ~1, 0);
            const unsigned sel = 2u * ((unsigned)delta & 1u);
            const unsigned* const rw =
                (const unsigned*)(bstrip + (ln & 31u) * 144u) + (delta >> 1) + 2 * (15 - (int)(ln >> 5));
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const unsigned* const d = rw - 2 * (8 * s2 + 2 * jj);
                    const unsigned d0 = d[0], d1 = d[1], d2 = d[2];
                    const unsigned x0 = __builtin_amdgcn_alignbyte(d1, d0, sel);
                    const unsigned x1 = __builtin_amdgcn_alignbyte(d2, d1, sel);
                    w[s2][jj][0] = __uint_as_float(x0 << 16);
                    w[s2][jj][1] = __uint_as_float(x0 & 0xFFFF0000u);
                    w[s2][jj][2] = __uint_as_float(x1 << 16);
                    w[s2][jj][3] = __uint_as_float(x1 & 0xFFFF0000u);
                }
        } else {
            // chunk k = 15 - 8 s - 2 jj - hh of row qi (distances R - 32 s - 8 jj - 4 hh - 3 ..)
            // sits at slot k ^ (qi % 16) = (15 ^ hh ^ (qi % 16)) ^ (8 s + 2 jj)
            const unsigned rb = (ln & 31u) * 256u + 16u * (15u ^ (ln >> 5) ^ (ln & 15u));
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    w[s2][jj] = *(const f32x4*)(bstrip + (rb ^ (unsigned)(16 * (8 * s2 + 2 * jj))));
        }
        if (code & BC_ROWS) {
            // A 16-byte run that reaches past the end of the (batch row, head) block reads as zeros
            // in full, entries inside the block included.  A row whose runs may reach that far
            // (its first needed entry s0 plus the run span passes Sq E) reads its entries one by
            // one at their exact offsets instead; the span grows with the row, so the wave's last
            // row decides whether any row does.
            constexpr int SPAN = PROF_BF16 ? 72 : BN;
            const int last = min(i0 + BM, p.Sq) - 1;
            const int lim = p.Sq * p.E;
            if (last * p.E + (qlo + last - i0) - j0t - (BN - 1) + SPAN > lim) {
                const int s0r = i * p.E + gi - j0t - (BN - 1);
                if (i < p.Sq && s0r + SPAN > lim) {
                    const unsigned rd = (unsigned)(gi - 4 * hh - j0t);
                    const unsigned rowoff = (unsigned)i * (unsigned)p.E;
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const unsigned r = rd - (unsigned)(32 * s2 + 8 * jj + (e ^ 3));
                                const unsigned off = opaque(r < (unsigned)p.E ? (rowoff + r) * PE : 0xFFFFFFF0u);
                                if constexpr (PROF_BF16)
                                    w[s2][jj][e] = __uint_as_float(
                                        (unsigned)__builtin_amdgcn_raw_buffer_load_b16(prsrc, (int)off, 0, 0) << 16);
                                else
                                    w[s2][jj][e] = __uint_as_float(
                                        __builtin_amdgcn_raw_buffer_load_b32(prsrc, (int)off, 0, 0));
                            }
                }
            }
        }
        if (code & BC_FAR) {
            // distances outside [0, E) take no bias
            const unsigned rd = opaque((unsigned)(gi - 4 * hh - j0t));
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const unsigned r = rd - (unsigned)(32 * s2 + 8 * jj + (e ^ 3));
                        w[s2][jj][e] = r < (unsigned)p.E ? w[s2][jj][e] : 0.0f;
                    }
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    a[s2][4 * jj + e] = __builtin_fmaf(w[s2][jj][e], INV_SCALE, a[s2][4 * jj + e]);
    };

    // ---- profile rows formed in-kernel (REL > 0).  profiles[b, h, i, r] =
    // sum_c rfeat[b, i, h, c] * table[r, c] (the table slice of head h).  For
    // a tile with keys j0 .. j0 + 63 the wave needs distances rho0 .. rho0 + 94,
    // rho0 = qlo - j0 - 63: P[rho', n] = table[rho0 + rho'] . rfeat[i0 + n] is
    // three 32 x 32 MFMA blocks (table rows on M, queries on N), and row n of
    // the strip holds P[n .. n + 63, n] (distance rho0 + n + e at entry e).
    // Table rows outside [0, E) read as 0 (range check), so distances outside
    // [0, E) take bias 0 with no further test.
    const __amdgpu_buffer_rsrc_t trsrc = uniform_rsrc(p.table + (REL ? h * p.t_hs : 0),
                                                      REL ? (size_t)p.E * REL * 2 : 0);
    typedef int i32x4_t __attribute__((ext_vector_type(4)));
    // Does this wave take bias on tile d (some distance below E)?
    auto rel_needed = [&](const TileDesc& d) -> bool {
        return REL > 0 && p.E > 0 && d.kt >= 0 && d.kt <= kt_hi && d.my_cls != TILE_SKIP &&
               qlo - (d.kt * BN + BN - 1) < p.E;
    };
    // A operands: lane (row m = lane % 32, half hh) of block s, k-step kk holds
    // table[rho0 + 32 s + m, 16 kk + 8 hh + 0..7]
    auto load_table = [&](int j0t, bf16x8 (&ta)[3][NRK]) {
        const unsigned ln = opaque((unsigned)lane);
        const unsigned row = (unsigned)(qlo - j0t - (BN - 1)) + (ln & 31u);
        const unsigned base = (row * (unsigned)REL + 8u * (ln >> 5)) * 2u;
#pragma unroll
        for (int s3 = 0; s3 < 3; ++s3)
#pragma unroll
            for (int kk = 0; kk < NRK; ++kk) {
                // (the whole offset travels in the range-checked register)
                const unsigned off = opaque(base + (unsigned)(32 * s3 * REL + 16 * kk) * 2u);
                const i32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(trsrc, (int)off, 0, 0);
                ta[s3][kk] = __builtin_bit_cast(bf16x8, x);
            }
    };
    // P of the tile into this wave's strip (row n at SROW n; no swizzle).
    // Lane (n, hh) holds P[32 s + 8 jj + 4 hh + e, n] of block s.  Block 1
    // (rows 32 .. 63) always lies in the band n .. n + 63; of blocks 0 and 2,
    // exactly one value of each pair (x, x + 64) does: x >= n takes block 0
    // (entry x - n), else block 2 (entry x + 64 - n).
    auto form_strip = [&](const bf16x8 (&ta)[3][NRK]) {
        f32x16 pc[3];
#pragma unroll
        for (int s3 = 0; s3 < 3; ++s3) {
            pc[s3] = f32x16{};
#pragma unroll
            for (int kk = 0; kk < NRK; ++kk)
                pc[s3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[s3][kk], rreg[kk], pc[s3], 0, 0, 0);
        }
        const unsigned ln = opaque((unsigned)lane);
        const unsigned n = ln & 31u, h4 = 4u * (ln >> 5);
        float* const row = (float*)(bstrip + (SROW - 4) * n + 4 * h4);   // entry x - n of row n at + 4 x
        const int nn = (int)n - (int)h4;                                  // x >= n  <=>  8 jj + e >= nn
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int xl = 8 * jj + e;                                // x = xl + 4 hh
                row[32 + xl] = pc[1][4 * jj + e];
                const bool lo = xl >= nn;
                const float v = lo ? pc[0][4 * jj + e] : pc[2][4 * jj + e];
                row[xl + (lo ? 0 : 64)] = v;
            }
    };
    // Adds the strip (formed for this tile) times sqrt(D) to the accumulators.
    auto bias_add_formed = [&](f32x16* a) {
        // chunk k = 15 - 8 s - 2 jj - hh of row qi at SROW qi + 16 k
        const unsigned ln = opaque((unsigned)lane);
        const char* rb = bstrip + (ln & 31u) * (unsigned)SROW + 16u * (15u - (ln >> 5));
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const f32x4 w = *(const f32x4*)(rb - 16 * (8 * s2 + 2 * jj));
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    a[s2][4 * jj + e] = __builtin_fmaf(w[e], INV_SCALE, a[s2][4 * jj + e]);
            }
    };

    // Software pipeline, per 64-key tile t: the DMA of the next live tile is
    // issued first; S^T = K Q^T of both 32-key halves runs as two interleaved
    // MFMA chains; tile t's bias (loaded during tile t - 1) is added and the
    // bias loads of tile t + 1 go out, staying in flight across the
    // end-of-tile barrier, which waits for the DMA alone.  Then the PV product
    // of tile t - 1 runs on the matrix cores while the softmax of tile t runs
    // on the vector units: one softmax step covers the 64 keys.
    TileDesc cur = next_live();
    int bcode = 0;   // bias code of the current tile (load_bias)
    {
        // V buffer 2 stands for the tile before the first: zeros
        f32x4* z = (f32x4*)(smem + V_OFF + 2 * VBYTES);
        for (int t = tid; t < VBYTES / 16; t += 64 * NW) z[t] = f32x4{};
    }
    // Tiles before kt_split carry no bias for any wave of the workgroup (every
    // distance of the workgroup's first query column to the tile's last key is
    // at least E); they run a loop body without the bias code.
    const int qlo_wg = p.qoff + qb_first * BM;
    const int kt_split = p.E <= 0 ? INT_MAX : (qlo_wg - p.E - (BN - 1) >= 0 ? (qlo_wg - p.E - (BN - 1)) / BN + 1 : 0);
    if (cur.kt <= kt_hi) issue_tile(cur, 0, 0);
    wait_all_and_barrier();
    // The descriptor of the tile after the current one is read one tile
    // ahead, before the barrier that ends the previous tile, so that its LDS
    // read is not waited for at the start of the tile.
    TileDesc nxt_pre = next_live();
    int kbuf = 0, vbuf = 0, vprev = 2;
    f16x8 pbp[4];   // P^T of the previous tile (zero when this wave did not compute it)
#pragma unroll
    for (int c = 0; c < 4; ++c) pbp[c] = f16x8{};
    constexpr int KHALF = (32 / L::RPI) * L::KGP;   // +32 keys in the K buffer
    // One tile of the pipeline; WB: with the bias code.
    auto step = [&](auto with_bias) {
        constexpr bool WB = decltype(with_bias)::value;
        const TileDesc nxt = nxt_pre;
        const int j0 = cur.kt * BN;
        const int vnext = vbuf == 2 ? 0 : vbuf + 1;

        // (after the last tile the current one is fetched again into the free
        // buffers, which nothing reads, so that every iteration issues the same
        // memory instructions)
        // (REL > 0: the table operands of this tile go out before the DMA of
        // the next one, so that waiting for them leaves that DMA in flight)
        bf16x8 tab[3][NRK];
        bool formed = false;
        if constexpr (WB && REL > 0) {
            formed = rel_needed(cur);
            if (formed) load_table(j0, tab);
        }
        // ---- S^T = K Q^T for keys j0 .. j0 + 63: two independent chains.  The
        // operands of k-step kk + 2 are read from LDS while k-step kk multiplies;
        // those of the first two k-steps go out before the next tile's DMA, whose
        // address set-up then hides their latency.
        const char* kb = smem + K_OFF + kbuf * KBYTES;
        auto kread = [&](int kk, int h2) -> bf16x8 {
            return *(const bf16x8*)(kb + ((kk & 1) ? kbase_odd : kbase_even) + 32 * kk + h2 * KHALF);
        };
        bf16x8 ka[NKK][2];
        ka[0][0] = kread(0, 0);
        ka[0][1] = kread(0, 1);
        ka[1][0] = kread(1, 0);
        ka[1][1] = kread(1, 1);
        asm volatile("" ::: "memory");
        issue_tile(nxt.kt <= kt_hi ? nxt : cur, kbuf ^ 1, vnext);
        asm volatile("" ::: "memory");
        const char* vbp = smem + V_OFF + vprev * VBYTES;
        // V^T chunk 2 c + hh of row qi sits at slot (2 c + hh) ^ vt_swz(qi) = (hh ^ vt_swz(qi)) ^ 2 c
        const unsigned ln = opaque((unsigned)lane);   // (derived here, not held in registers)
        const unsigned vb = (ln & 31u) * 128u + 16u * ((ln >> 5) ^ (unsigned)vt_swz((int)(ln & 31u)));

        f32x16 acc[2];
        {
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                if (kk + 2 < NKK) {
                    ka[kk + 2][0] = kread(kk + 2, 0);
                    ka[kk + 2][1] = kread(kk + 2, 1);
                }
                acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk][0], qreg[kk], kk ? acc[0] : f32x16{}, 0, 0, 0);
                acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk][1], qreg[kk], kk ? acc[1] : f32x16{}, 0, 0, 0);
            }
#pragma unroll
            for (int kk = 0; kk + 2 < NKK; ++kk) {
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // LDS reads
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);       // MFMA
        }
        // operands of step 0 of the previous tile's PV product (read while the
        // chains above finish)
        f16x8 avs[4][NDB];   // operands of the four steps (each step's own registers)
#pragma unroll
        for (int db = 0; db < NDB; ++db) avs[0][db] = *(const f16x8*)(vbp + vb + db * 32 * 128);
        // ---- + bias * sqrt(D) (nothing on tiles this wave skips); the bias
        // registers / strip then take the next tile's
        int ncode = 0;   // bias code of the next tile
        if constexpr (WB && REL > 0) {
            if (formed) {
                wait_vm_keep(N_KV_DMA);
                form_strip(tab);
                __builtin_amdgcn_s_waitcnt(WAIT_LGKM);   // this wave's strip writes are done
                bias_add_formed(acc);
                __builtin_amdgcn_s_waitcnt(WAIT_LGKM);   // and read, before the next tile rewrites it
            }
        } else if constexpr (WB) {
            bias_add_tile(bcode, j0, acc);
            asm volatile("" ::: "memory");
            ncode = load_bias(nxt);
            asm volatile("" ::: "memory");
        }

        // ---- mask (every key of a tile this wave skips is masked: no allowed
        // pair).  Element (jj, e) of half s is key j0 + 32 s + 8 jj + 4 hh + (e ^ 3).
        if (cur.my_cls != TILE_FULL) {
            const int* ca = (const int*)(smem + CA_OFF + kbuf * BN * 4);
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int kl = 32 * s2 + 8 * jj + 4 * hh;
                    const i32x4 c4 = *(const i32x4*)(ca + kl);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (!key_visible(gi_eff, a_q, j0 + kl + (e ^ 3), c4[e ^ 3], wlim))
                            acc[s2][4 * jj + e] = -INFINITY;
                }
        }

        // ---- the softmax frame.  The running frame m (log2 units) only has to
        // keep this tile's fp16 weights e^{z - m} in range; it is not moved to
        // each tile's row max.  A row takes its first frame from the first tile
        // with a finite logit when it has no sink (its output, denominator and
        // previous weights are still zero then); afterwards the frame moves
        // only when a weight would leave the fp16 range, which the row's partial
        // sums show after the fact (below).
        auto row_max = [&]() -> float {
            float mx = -INFINITY;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                mx = fmaxf(mx, acc[0][t]);
                mx = fmaxf(mx, acc[1][t]);
            }
            return half_max(mx * p.c_log2);
        };
        if (__builtin_amdgcn_ballot_w64(m == -INFINITY) != 0) {
            const float mx = row_max();
            if (m == -INFINITY) m = mx;
        }
        float m_use = (m == -INFINITY) ? 0.0f : m;

        // ---- the previous tile's O^T += V^T P^T in four steps, with this
        // tile's weights P^T on the vector units meanwhile.  pb[c] holds keys
        // 16 c + ... in the order of V^T's staged rows.
        // Without bias, this tile's weights replace the previous tile's in pbp,
        // step by step, once the products that read them have been issued (no
        // copy closes the iteration); the bias loop keeps its own array
        f16x8 pbl[4];
        f16x8 (&pb)[4] = *(WB ? &pbl : &pbp);
        float ls0 = 0.0f, ls1 = 0.0f;
        auto make_p = [&](int c) {
#pragma unroll
            for (int t = 0; t < 8; ++t)
                pb[c][t] = (_Float16)__builtin_amdgcn_exp2f(
                    __builtin_fmaf(acc[c >> 1][8 * (c & 1) + t], p.c_log2, -m_use));
            // the denominator sums the fp16-rounded weights the PV product uses
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2) {
                const half2_t w2 = half2_t{pb[c][2 * q2], pb[c][2 * q2 + 1]};
                if (q2 & 1) ls1 = __builtin_amdgcn_fdot2(w2, half2_t{(_Float16)1.0f, (_Float16)1.0f}, ls1, false);
                else ls0 = __builtin_amdgcn_fdot2(w2, half2_t{(_Float16)1.0f, (_Float16)1.0f}, ls0, false);
            }
        };
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            // the operands of step c + 1 are read while step c multiplies
            if (c < 3) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    avs[c + 1][db] = *(const f16x8*)(vbp + (vb ^ (32u * (c + 1))) + db * 32 * 128);
            }
            if constexpr (WB) make_p(c);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(avs[c][db], pbp[c], oacc[db], 0, 0, 0);
            if constexpr (!WB) make_p(c);
            if (c < 3) __builtin_amdgcn_sched_group_barrier(0x100, NDB, 0);     // LDS reads
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // VALU
            }
            if constexpr (WB) __builtin_amdgcn_sched_barrier(0);   // each step is scheduled on its own
        }
        // (the weights are pinned here, so that the compiler does not sink
        // their computation below the MFMAs it is meant to overlap)
#pragma unroll
        for (int c = 0; c < 4; ++c) pin(pb[c]);
        // A lane's 32 weights summing below 2^15 are each below 2^15, inside
        // fp16's range.  Otherwise (or a NaN) the frame moves to the row max:
        // the output so far (all of the previous tile's product included) and
        // the denominator are rescaled and this tile's weights are formed again.
        if (__builtin_amdgcn_ballot_w64(!(ls0 + ls1 < FRAME_LIMIT)) != 0) {
            const float mx = row_max();
            const float m_new = fmaxf(m, mx);
            // (rows of the wave whose frame stays put, one still unset among
            // them, keep their sums: e^{-inf - (-inf)} would be a NaN)
            const float alpha = m_new > m ? __builtin_amdgcn_exp2f(m - m_new) : 1.0f;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int t = 0; t < 16; ++t) oacc[db][t] *= alpha;
            m = m_new;
            m_use = (m_new == -INFINITY) ? 0.0f : m_new;
            ls0 = 0.0f;
            ls1 = 0.0f;
#pragma unroll
            for (int c = 0; c < 4; ++c) make_p(c);
        }
        l += ls0 + ls1;
        if constexpr (WB) {
#pragma unroll
            for (int c = 0; c < 4; ++c) pbp[c] = pb[c];
        }

        nxt_pre = next_live();   // (the tile after nxt)
        // this wave's part of the next tile's DMA has landed (the bias loads
        // issued after it may still be in flight); then every wave's has
        wait_dma_and_barrier(WB ? bias_loads(ncode) : 0);
        bcode = ncode;
        kbuf ^= 1;
        vprev = vbuf;
        vbuf = vnext;
        cur = nxt;
        };
    while (cur.kt <= kt_hi && cur.kt < kt_split) step(std::false_type{});
    // the first tile that may carry bias: its loads overlap its own QK^T
    if (REL == 0 && cur.kt <= kt_hi) bcode = load_bias(cur);
    while (cur.kt <= kt_hi) step(std::true_type{});
    // ---- the last tile's O^T += V^T P^T
    {
        const char* vbp = smem + V_OFF + vprev * VBYTES;
        const unsigned ln = opaque((unsigned)lane);
        const unsigned vb = (ln & 31u) * 128u + 16u * ((ln >> 5) ^ (unsigned)vt_swz((int)(ln & 31u)));
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    *(const f16x8*)(vbp + (vb ^ (32u * c)) + db * 32 * 128), pbp[c], oacc[db], 0, 0, 0);
    }

    // ---- epilogue.  fp32 rows leave through this wave's bias strip, free now:
    // the wave writes its normalised O^T there as rows of D / 2 columns (16-byte
    // chunks XOR-swizzled by row), reads them back a row run per 16 lanes and
    // stores 4 whole rows of 256 bytes per instruction (the accumulator layout
    // would store 32 rows x 32 bytes).  Half of D per pass (8 KB).
    const float l_tot = half_sum(l);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (!p.out_bf16) {
        __builtin_amdgcn_s_waitcnt(WAIT_VM_LGKM);   // no DMA into the strip outstanding, no read of it
        const int rows_here = qb < p.nQB ? min(BM, p.Sq - i0) : 0;
        const unsigned ln = opaque((unsigned)lane);
        float* const orow = (float*)p.out + b * p.o_bs + (long long)i0 * p.o_ts + h * p.o_hs;
#pragma unroll
        for (int hp = 0; hp < NDB / 2; ++hp) {
            // lane (qi, hh) holds columns 64 hp + 32 dbl + 8 jj + 4 hh + 0..3 of row qi: chunk 8 dbl + 2 jj + hh
#pragma unroll
            for (int dbl = 0; dbl < 2; ++dbl)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    f32x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = oacc[2 * hp + dbl][4 * jj + e] * inv;
                    const unsigned c = 8u * dbl + 2u * jj + (ln >> 5);
                    *(f32x4*)(bstrip + (ln & 31u) * 256u + 16u * (c ^ (ln & 15u))) = w;
                }
            // instruction u: row 4 u + lane / 16, chunk lane % 16
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const unsigned r = 4u * u + (ln >> 4), c = ln & 15u;
                const f32x4 w = *(const f32x4*)(bstrip + r * 256u + 16u * (c ^ (r & 15u)));
                if ((int)r < rows_here) *(f32x4*)(orow + (long long)r * p.o_ts + 64 * hp + 4 * (int)c) = w;
            }
            __builtin_amdgcn_s_waitcnt(WAIT_LGKM);   // read back before the next pass rewrites the strip
        }
    }
    if (!qin) return;
    if (p.out_bf16) {
        const long long oo = b * p.o_bs + (long long)i * p.o_ts + h * p.o_hs;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                bf16x4 wb;
#pragma unroll
                for (int e = 0; e < 4; ++e) wb[e] = (__bf16)(oacc[db][4 * jj + e] * inv);   // round to nearest even
                *(bf16x4*)((__bf16*)p.out + oo + 32 * db + 8 * jj + 4 * hh) = wb;
            }
    }
    if (hh == 0 && p.lse) {
        float lse;
        if (!qreal) lse = sig;
        else if (l_tot > 0.0f) lse = (m + log2f(l_tot)) * LN2;
        else lse = -INFINITY;
        p.lse[b * p.l_bs + (long long)i * p.l_ts + h * p.l_hs] = lse;
    }
}

// ---------------------------------------------------------------------------
// Value staging.  One workgroup of D threads per (batch row, K/V head, 64-key
// tile): v (bf16) -> V^T (fp16), the keys of each row in vt_slot order, 0 at
// keys that are not real or lie past Sk (a masked key's weight 0 never meets
// a value fp16 cannot hold).  A real value outside +-65504 (or not finite) has
// no fp16 form: it is written as NaN, so that the rows that use it come out
// NaN instead of silently wrong, and the tile's byte in `bad` is set (0
// otherwise; every tile writes its byte on every call).  Thread (slot group
// sg, dim chunk dc) loads the 8 keys of output slots 8 sg .. 8 sg + 7 at dims
// 8 dc .. 8 dc + 7, transposes the 8 x 8 block in registers and writes 8 rows
// of 16 bytes.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(D) void stage_values_kernel(const __bf16* __restrict__ v,
                                                         const uint8_t* __restrict__ key_valid,
                                                         int Sk, int Hkv, int nKT, long long v_bs,
                                                         long long v_ts, long long v_hs,
                                                         _Float16* __restrict__ vt, uint8_t* __restrict__ bad)
{
    constexpr int CH = D / 8;                 // 16-byte chunks per key row
    const int t = blockIdx.x;                 // ((b * Hkv + g) * nKT + kt)
    const int kt = t % nKT;
    const int g = (t / nKT) % Hkv;
    const int b = t / (nKT * Hkv);
    const int sg = threadIdx.x / CH, dc = threadIdx.x % CH;
    // every row and its validity byte are loaded before any is used (one
    // memory round trip, not one per row)
    // (keys past Sk load key Sk - 1, branch-free, and are dropped below)
    bf16x8 xr[8];
    int ok[8];
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
        // slot 8 sg + tt holds key 16 (sg / 2) + 8 (tt / 4) + 4 (sg % 2) + ((tt % 4) ^ 3)
        const int key = 16 * (sg >> 1) + 8 * (tt >> 2) + 4 * (sg & 1) + ((tt & 3) ^ 3);
        const int j = min(kt * BN + key, Sk - 1);
        xr[tt] = *(const bf16x8*)(v + b * v_bs + j * v_ts + g * v_hs + 8 * dc);
        ok[tt] = key_valid[(size_t)b * Sk + j];
    }
    f16x8 rows[8];
    int out_of_range = 0;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
        const int key = 16 * (sg >> 1) + 8 * (tt >> 2) + 4 * (sg & 1) + ((tt & 3) ^ 3);
        f16x8 y = f16x8{};
        if (ok[tt] && kt * BN + key < Sk) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float f = (float)xr[tt][e];
                const bool fits = fabsf(f) <= 65504.0f;   // false for NaN and infinities too
                out_of_range |= !fits;
                y[e] = fits ? (_Float16)f : (_Float16)__builtin_nanf("");
            }
        }
        rows[tt] = y;
    }
    out_of_range = __syncthreads_or(out_of_range);
    if (threadIdx.x == 0) bad[t] = (uint8_t)(out_of_range != 0);
    _Float16* dst = vt + (size_t)t * D * BN;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        f16x8 o;
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) o[tt] = rows[tt][e];
        *(f16x8*)(dst + (8 * dc + e) * BN + 8 * sg) = o;
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

// One thread per (batch row, query, key): the same predicate as the attention
// kernel's masked tiles, written as one byte.
__global__ void debug_mask_kernel(const uint8_t* __restrict__ valid, const uint8_t* __restrict__ key_valid,
                                  const int32_t* __restrict__ positions, const int32_t* __restrict__ key_positions,
                                  int window, int qoff, int Sq, int Sk, size_t n, uint8_t* __restrict__ mask)
{
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n) return;
    const int j = (int)(idx % Sk);
    const size_t qrow = idx / Sk;               // b * Sq + i
    const int b = (int)(qrow / Sq), i = (int)(qrow % Sq);
    const int gi = qoff + i;
    const bool qreal = valid[qrow] != 0;
    const int a_q = qreal ? (positions ? gi - positions[qrow] : 0) : 0;
    const size_t o = (size_t)b * Sk + j;
    const int c = key_valid[o] ? (key_positions ? j - key_positions[o] : 0) : INT_MIN;
    const unsigned wlim = window > 0 ? (unsigned)window : 0x80000000u;
    mask[idx] = key_visible(qreal ? gi : -1, a_q, j, c, wlim) ? 1 : 0;
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

}  // namespace

// Workspace of attn_fwd_noalloc: one copy per GPU, at that GPU's own address,
// held from the first use on the GPU until the process ends.  Host code never
// passes this name to a kernel or a copy (on the host it only stands for the
// symbol); it uses the device address hipGetSymbolAddress returns for it.
static __device__ __align__(256) unsigned char scratch[INKATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};   // device address of `scratch`, per device

// Device address of the current device's scratch (looked up once per device,
// with that device current).
int scratch_address(void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(INKATTN_ERR_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= MAX_DEVICES) return fail(INKATTN_ERR_LAUNCH, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(INKATTN_ERR_LAUNCH, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return INKATTN_OK;
}

}  // namespace

namespace inkattn __attribute__((visibility("hidden"))) {

thread_local char g_last_error[512] = "";

void clear_error() { g_last_error[0] = '\0'; }

int fail(int status, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }


// Workspace layout: [tile summaries][key start columns, int32 B*Sk][values in fp16, B*Sk*Hkv*D],
// the first two parts each rounded up to 256 bytes.  summaries_bytes covers the
// first two parts (what the pre-pass writes).
size_t round256(size_t x) { return (x + 255) / 256 * 256; }
size_t tile_summary_bytes(int B, int Sq, int Sk)
{
    const size_t nq = (size_t)B * ceil_div(Sq, BM);
    const size_t nk = (size_t)B * ceil_div(Sk, BN);
    return round256((nq + nk) * sizeof(TileSummary));
}
size_t summaries_bytes(int B, int Sq, int Sk)
{
    return tile_summary_bytes(B, Sq, Sk) + round256((size_t)B * ceil_div(Sk, BN) * BN * sizeof(int));
}

size_t values_bytes(int B, int Sk, int Hkv, int D)
{
    return (size_t)B * Hkv * ceil_div(Sk, BN) * BN * D * sizeof(_Float16);
}

size_t value_flags_bytes(int B, int Sk, int Hkv) { return round256((size_t)B * Hkv * ceil_div(Sk, BN)); }

size_t fwd_workspace_bytes(int B, int Sq, int Sk, int Hkv, int D)
{
    return summaries_bytes(B, Sq, Sk) + values_bytes(B, Sk, Hkv, D) + value_flags_bytes(B, Sk, Hkv);
}

int check_tile_counts(int B, int Sq, int Sk, int Hq, int Hkv)
{
    const long long nQB = ceil_div(Sq, BM), nKT = ceil_div(Sk, BN);
    if ((long long)B * (nQB + nKT) >= (1LL << 31)) return fail(INKATTN_ERR_SHAPE, "too many tiles");
    if ((long long)B * Hkv * nKT >= (1LL << 31)) return fail(INKATTN_ERR_SHAPE, "v too large");
    if ((long long)B * Hq * nQB >= (1LL << 31)) return fail(INKATTN_ERR_SHAPE, "grid too large");
    return INKATTN_OK;
}

// Defaults of the optional arguments and the checks shared by every entry point.

int resolve_mask_args(const uint8_t* valid, const uint8_t* key_valid, const int32_t* positions,
                      const int32_t* key_positions, int64_t query_offset, int B, int Sq, int Sk,
                      MaskArgs* outa)
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

int check_workspace(void* workspace, size_t workspace_bytes, size_t need)
{
    if (!workspace || workspace_bytes < need)
        return fail(INKATTN_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
    if (!aligned(workspace, 16)) return fail(INKATTN_ERR_ALIGN, "workspace not 16-byte aligned");
    return INKATTN_OK;
}

int launch_summaries(const uint8_t* valid, const int32_t* positions, const uint8_t* key_valid,
                     const int32_t* key_positions, int qoff, int B, int Sq, int Sk,
                     void* workspace, hipStream_t st)
{
    TileSummary* qsum = (TileSummary*)workspace;
    TileSummary* ksum = qsum + (size_t)B * ceil_div(Sq, BM);
    int* kanchor = (int*)((char*)workspace + tile_summary_bytes(B, Sq, Sk));
    const int nQB = ceil_div(Sq, BM), nKT = ceil_div(Sk, BN);
    const long long waves = (long long)B * (nQB + nKT);
    if (waves == 0) return INKATTN_OK;
    if (waves >= (1LL << 31)) return fail(INKATTN_ERR_SHAPE, "too many tiles");
    const int blocks = (int)((waves + 3) / 4);
    hipLaunchKernelGGL(summarize_kernel, dim3(blocks), dim3(256), 0, st, valid, positions, qoff, Sq, nQB,
                       key_valid, key_positions, Sk, nKT, B, qsum, ksum, kanchor);
    return check_launch("summarize_kernel");
}

}  // namespace inkattn

namespace {

// Checks of attn_fwd / attn_fwd_planned that need no device access.
int check_fwd_args(const void* q, const void* k, const void* v, const void* profiles, int profiles_dtype,
                   const float* sink, int B, int Sq, int Sk, int Hq, int Hkv, int D, int E,
                   float* out, float* lse)
{
    if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
        return fail(INKATTN_ERR_SHAPE, "Hq=%d must be a positive multiple of Hkv=%d", Hq, Hkv);
    if (E < 1) return fail(INKATTN_ERR_SHAPE, "relative extent E=%d must be >= 1", E);
    if (D != 64 && D != 128) return fail(INKATTN_ERR_UNSUPPORTED, "head_dim %d not built (64, 128)", D);
    if (profiles_dtype != INKATTN_F32 && profiles_dtype != INKATTN_BF16)
        return fail(INKATTN_ERR_UNSUPPORTED, "profiles dtype %d unknown", profiles_dtype);
    const size_t nq_elems = (size_t)B * Sq * Hq * D;
    const size_t np_elems = (size_t)B * Hq * Sq * E;
    if (nq_elems >= (size_t(1) << 40) || np_elems >= (size_t(1) << 40))
        return fail(INKATTN_ERR_SHAPE, "tensor too large");
    if ((size_t)Sq * E * (profiles_dtype == INKATTN_F32 ? 4 : 2) >= (size_t(1) << 32))
        return fail(INKATTN_ERR_SHAPE, "one (batch row, head) block of profiles must stay below 4 GiB");
    if ((size_t)B * Sq == 0) return INKATTN_OK;
    if (!q || !profiles || !sink || !out || !lse) return fail(INKATTN_ERR_NULL, "q/profiles/sink/out/lse is NULL");
    if (Sk > 0 && (!k || !v)) return fail(INKATTN_ERR_NULL, "k or v is NULL");
    if (!aligned(q, 16) || (Sk > 0 && (!aligned(k, 16) || !aligned(v, 16))) || !aligned(out, 16))
        return fail(INKATTN_ERR_ALIGN, "q, k, v and out must be 16-byte aligned");
    if (!aligned(profiles, profiles_dtype == INKATTN_F32 ? 4 : 2) || !aligned(sink, 4) || !aligned(lse, 4))
        return fail(INKATTN_ERR_ALIGN, "profiles / sink / lse misaligned");
    return INKATTN_OK;
}

// Workgroup shape: NWAVES waves; heads per workgroup hpw divides G; hpw * tpw = NWAVES.
struct Shape {
    int nw, hpw, tpw;
};

Shape choose_shape(int G)
{
    Shape s;
    s.nw = NWAVES;
    s.hpw = (G % 8 == 0) ? 8 : (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
    s.tpw = s.nw / s.hpw;
    return s;
}

template <int D, bool PB, int REL>
void launch_fwd(const Shape& sh, dim3 grid, hipStream_t st, const FwdParams& p)
{
    (void)sh;
    hipLaunchKernelGGL((attn_fwd_kernel<D, PB, NWAVES, REL>), grid, dim3(64 * NWAVES), 0, st, p);
}

// Positions for the generic flex forward, one workgroup per batch row: a
// token's position counts from the start of its block, where blocks end after
// every token equal to eos (when tokens is given) and, with fixed > 0, also
// start at every multiple of fixed.  Also writes nones bytes of 1 (token
// validity: every token is real).
__global__ __launch_bounds__(1024) void flex_positions_kernel(const int32_t* __restrict__ tokens, int eos,
                                                              int fixed, int S, int32_t* __restrict__ pos,
                                                              uint8_t* __restrict__ ones, size_t nones)
{
    constexpr int PER = 8;                       // tokens per thread and pass
    constexpr int NWV = 1024 / 64;               // waves
    __shared__ int wmax[2][NWV];
    const int b = blockIdx.x, t = threadIdx.x;
    const int lane = t & 63, wv = t >> 6;
    for (size_t u = (size_t)b * 1024 + t; u < nones; u += (size_t)gridDim.x * 1024) ones[u] = 1;
    if (!pos) return;
    const int32_t* tk = tokens ? tokens + (size_t)b * S : nullptr;
    int32_t* ps = pos + (size_t)b * S;
    int carry = 0;                               // start column after the last eos so far
    for (int base = 0; base < S; base += 1024 * PER) {
        // token base + 1024 c + t of chunk c: all loads go out first (coalesced)
        int is_eos[PER];
#pragma unroll
        for (int c = 0; c < PER; ++c) {
            const int u = base + 1024 * c + t;
            is_eos[c] = (tk && u < S) ? (tk[u] == eos) : 0;
        }
#pragma unroll
        for (int c = 0; c < PER; ++c) {
            const int u = base + 1024 * c + t;
            // running max of (eos column + 1) over the chunk's tokens up to
            // this one: inclusive within the wave by shuffles, then over the
            // waves before through LDS (two slots: one barrier per chunk)
            int inc = is_eos[c] ? u + 1 : 0;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int other = __shfl_up(inc, d, 64);
                if (lane >= d) inc = max(inc, other);
            }
            if (lane == 63) wmax[c & 1][wv] = inc;
            __syncthreads();
            int before = carry, chunk_max = carry;
            for (int w = 0; w < NWV; ++w) {
                const int x = wmax[c & 1][w];
                if (w < wv) before = max(before, x);
                chunk_max = max(chunk_max, x);
            }
            const int prev = __shfl_up(inc, 1, 64);   // inclusive value of the lane before
            const int start = max(before, lane > 0 ? prev : 0);   // after the last eos before u
            if (u < S) {
                const int st = fixed > 0 ? max(start, (u / fixed) * fixed) : start;
                ps[u] = u - st;
            }
            carry = chunk_max;
        }
    }
}

// Launches the fp16 value staging for v with element strides (batch row,
// key, head) into the workspace (values, then one flag byte per staged tile).
int launch_stage(const __bf16* v, const uint8_t* key_valid, int B, int Sq, int Sk, int Hkv, int D, long long v_bs,
                 long long v_ts, long long v_hs, void* workspace, hipStream_t st)
{
    const size_t tiles = (size_t)B * Hkv * ceil_div(Sk, BN);
    if (tiles == 0) return INKATTN_OK;   // (the kernel reads key Sk - 1: Sk >= 1 from here on)
    if (tiles >= (size_t(1) << 31)) return fail(INKATTN_ERR_SHAPE, "v too large");
    _Float16* v16 = (_Float16*)((char*)workspace + summaries_bytes(B, Sq, Sk));
    uint8_t* bad = (uint8_t*)v16 + values_bytes(B, Sk, Hkv, D);
    if (D == 128)
        hipLaunchKernelGGL(stage_values_kernel<128>, dim3((unsigned)tiles), dim3(128), 0, st, v, key_valid, Sk, Hkv,
                           ceil_div(Sk, BN), v_bs, v_ts, v_hs, v16, bad);
    else
        hipLaunchKernelGGL(stage_values_kernel<64>, dim3((unsigned)tiles), dim3(64), 0, st, v, key_valid, Sk, Hkv,
                           ceil_div(Sk, BN), v_bs, v_ts, v_hs, v16, bad);
    return check_launch("stage_values_kernel");
}

struct Strides {
    long long bs, ts, hs;   // elements between batch rows, tokens, heads
};

// In-kernel profile rows (attn_fwd_relproj): relative features and table.
struct RelArgs {
    const void* rfeat = nullptr;
    const void* table = nullptr;
    int d_rel = 0;                 // 0: profiles are read
    long long r_bs = 0, r_ts = 0, r_hs = 0, t_hs = 0;
};

// Launches the attention kernel over a planned and staged workspace.
int run_forward(const void* q, const void* k, void* workspace, const void* profiles, int profiles_dtype,
                const float* sink, const uint8_t* valid, const MaskArgs& ma, const int32_t* positions, int window,
                int query_offset, int B, int Sq, int Sk, int Hq, int Hkv, int D, int E, void* out, int out_bf16,
                float* lse, Strides qs, Strides ks, Strides os, Strides ls, Strides ss, float c_log2,
                hipStream_t st, const RelArgs& rel = RelArgs{})
{
    const int nQB = ceil_div(Sq, BM), nKT = ceil_div(Sk, BN);
    const Shape sh = choose_shape(Hq / Hkv);

    FwdParams p;
    p.q = (const __bf16*)q;
    p.k = (const __bf16*)k;
    p.v16 = (const _Float16*)((const char*)workspace + summaries_bytes(B, Sq, Sk));
    p.profiles = profiles;
    p.sink = sink;
    p.valid = valid;
    p.key_valid = ma.key_valid;
    p.positions = positions;
    p.key_positions = ma.key_positions;
    p.qsum = (const TileSummary*)workspace;
    p.ksum = p.qsum + (size_t)B * nQB;
    p.kanchor = (const int*)((const char*)workspace + tile_summary_bytes(B, Sq, Sk));
    p.out = out;
    p.lse = lse;
    p.q_bs = qs.bs; p.q_ts = qs.ts; p.q_hs = qs.hs;
    p.k_bs = ks.bs; p.k_ts = ks.ts; p.k_hs = ks.hs;
    p.o_bs = os.bs; p.o_ts = os.ts; p.o_hs = os.hs;
    p.l_bs = ls.bs; p.l_ts = ls.ts; p.l_hs = ls.hs;
    p.s_bs = ss.bs; p.s_ts = ss.ts; p.s_hs = ss.hs;
    p.out_bf16 = out_bf16;
    p.B = B; p.Sq = Sq; p.Sk = Sk; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv; p.E = E;
    p.window = window;
    p.qoff = query_offset;
    p.hpw = sh.hpw;
    p.tpw = sh.tpw;
    p.nchunk = p.G / p.hpw;
    p.nQB = nQB; p.nQG = ceil_div(nQB, sh.tpw); p.nKT = nKT;
    p.c_log2 = c_log2;

    const size_t nblocks = (size_t)p.nQG * B * Hkv * p.nchunk;
    if (nblocks >= (size_t(1) << 31)) return fail(INKATTN_ERR_SHAPE, "grid too large");
    const dim3 grid((unsigned)nblocks);
    const bool pb = profiles_dtype == INKATTN_BF16;
    p.rfeat = (const __bf16*)rel.rfeat;
    p.table = (const __bf16*)rel.table;
    p.r_bs = rel.r_bs; p.r_ts = rel.r_ts; p.r_hs = rel.r_hs;
    p.t_hs = rel.t_hs;
    if (rel.d_rel == 16) {
        if (D == 128) launch_fwd<128, false, 16>(sh, grid, st, p);
        else launch_fwd<64, false, 16>(sh, grid, st, p);
    } else if (rel.d_rel == 32) {
        if (D == 128) launch_fwd<128, false, 32>(sh, grid, st, p);
        else launch_fwd<64, false, 32>(sh, grid, st, p);
    } else if (D == 128) {
        if (pb) launch_fwd<128, true, 0>(sh, grid, st, p);
        else launch_fwd<128, false, 0>(sh, grid, st, p);
    } else {
        if (pb) launch_fwd<64, true, 0>(sh, grid, st, p);
        else launch_fwd<64, false, 0>(sh, grid, st, p);
    }
    return check_launch("attn_fwd_kernel");
}

}  // namespace

extern "C" {

size_t attn_fwd_workspace_size(int B, int Sq, int Sk, int Hkv, int D)
{
    if (B <= 0 || Sq < 0 || Sk < 0 || Hkv < 0 || D < 0) return 0;
    return fwd_workspace_bytes(B, Sq, Sk, Hkv, D);
}

int attn_query_block(void) { return BM; }
int attn_key_tile(void) { return BN; }

size_t flex_attn_workspace_size(int B, int Sq, int Sk, int Hkv, int D)
{
    if (B <= 0 || Sq < 0 || Sk < 0 || Hkv < 0 || D < 0) return 0;
    return attn_fwd_workspace_size(B, Sq, Sk, Hkv, D) + round256((size_t)B * Sq * 4) +
           round256((size_t)B * std::max(Sq, Sk));
}

int flex_attn_fwd(const void* q, const void* k, const void* v, const float* sink_weights,
                  const int32_t* tokens, int32_t eos_id, int64_t fixed_block_size, int64_t sliding_window,
                  float scale, int B, int Sq, int Sk, int Hq, int Hkv, int D, void* out, float* lse,
                  void* workspace, size_t workspace_bytes, void* stream)
{
    g_last_error[0] = '\0';
    if (B < 0 || Sq < 0 || Sk < 0) return fail(INKATTN_ERR_SHAPE, "negative size");
    if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
        return fail(INKATTN_ERR_SHAPE, "Hq=%d must be a positive multiple of Hkv=%d", Hq, Hkv);
    if (D != 64 && D != 128) return fail(INKATTN_ERR_UNSUPPORTED, "head_dim %d not built (64, 128)", D);
    if (Sq >= (1 << 30) || Sk >= (1 << 30)) return fail(INKATTN_ERR_SHAPE, "sequence lengths must stay below 2^30");
    if ((size_t)B * Hq * Sq * D >= (size_t(1) << 40) || (size_t)Sk * D * 2 >= (size_t(1) << 32))
        return fail(INKATTN_ERR_SHAPE, "tensor too large");
    const bool blocks = tokens != nullptr || fixed_block_size > 0;
    if (blocks && Sq != Sk) return fail(INKATTN_ERR_SHAPE, "block masks need Sq == Sk (got %d, %d)", Sq, Sk);
    if (fixed_block_size >= (int64_t(1) << 31)) fixed_block_size = 0;
    if (sliding_window >= (int64_t(1) << 31) || sliding_window < 0) sliding_window = 0;
    if ((size_t)B * Sq == 0) return INKATTN_OK;
    if (!q || !out) return fail(INKATTN_ERR_NULL, "q or out is NULL");
    if (Sk > 0 && (!k || !v)) return fail(INKATTN_ERR_NULL, "k or v is NULL");
    if (!aligned(q, 16) || (Sk > 0 && (!aligned(k, 16) || !aligned(v, 16))) || !aligned(out, 16))
        return fail(INKATTN_ERR_ALIGN, "q, k, v and out must be 16-byte aligned");
    if ((sink_weights && !aligned(sink_weights, 4)) || (lse && !aligned(lse, 4)) || (tokens && !aligned(tokens, 4)))
        return fail(INKATTN_ERR_ALIGN, "sink_weights / lse / tokens misaligned");
    if (int rc = check_tile_counts(B, Sq, Sk, Hq, Hkv)) return rc;
    if (int rc = check_workspace(workspace, workspace_bytes, flex_attn_workspace_size(B, Sq, Sk, Hkv, D))) return rc;

    hipStream_t st = (hipStream_t)stream;
    char* ws = (char*)workspace;
    const size_t attn_ws = attn_fwd_workspace_size(B, Sq, Sk, Hkv, D);
    int32_t* pos = blocks ? (int32_t*)(ws + attn_ws) : nullptr;
    uint8_t* ones = (uint8_t*)(ws + attn_ws + round256((size_t)B * Sq * 4));
    const size_t nones = (size_t)B * std::max(Sq, Sk);
    MaskArgs ma;
    if (int rc = resolve_mask_args(ones, ones, pos, pos, 0, B, Sq, Sk, &ma)) return rc;
    // every check has run: from here on only launches
    hipLaunchKernelGGL(flex_positions_kernel, dim3((unsigned)B), dim3(1024), 0, st, tokens, (int)eos_id,
                       (int)fixed_block_size, Sq, pos, ones, nones);
    if (int rc = check_launch("flex_positions_kernel")) return rc;
    if (int rc = launch_summaries(ones, pos, ma.key_valid, ma.key_positions, 0, B, Sq, Sk, workspace, st)) return rc;
    if (Sk > 0) {
        const long long v_hs = (long long)Sk * D;
        if (int rc = launch_stage((const __bf16*)v, ones, B, Sq, Sk, Hkv, D, Hkv * v_hs, D, v_hs, workspace, st))
            return rc;
    }
    // scale: applied only without sink weights (the default head_dim^-0.5 otherwise)
    const double sc = (!sink_weights && scale > 0.0f) ? (double)scale : 1.0 / std::sqrt((double)D);
    const long long q_hs = (long long)Sq * D, k_hs = (long long)Sk * D;
    return run_forward(q, k, workspace, nullptr, INKATTN_F32, sink_weights, ones, ma, pos, (int)sliding_window, 0, B,
                       Sq, Sk, Hq, Hkv, D, 0, out, 1, lse, Strides{Hq * q_hs, D, q_hs},
                       Strides{Hkv * k_hs, D, k_hs}, Strides{Hq * q_hs, D, q_hs},
                       Strides{(long long)Hq * Sq, 1, Sq}, Strides{0, 0, 1},
                       (float)(sc * 1.4426950408889634), st);
}

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
    case INKATTN_ERR_RANGE: return "a value outside the supported range";
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
    if (int rc = resolve_mask_args(valid, key_valid, positions, key_positions, query_offset, B, Sq, Sk, &ma))
        return rc;
    if ((size_t)B * ((size_t)Sq + Sk) == 0) return INKATTN_OK;
    if (int rc = check_workspace(workspace, workspace_bytes, summaries_bytes(B, Sq, Sk))) return rc;
    return launch_summaries(valid, positions, ma.key_valid, ma.key_positions, (int)query_offset, B, Sq, Sk,
                            workspace, (hipStream_t)stream);
}

int attn_stage_values(const void* v, const uint8_t* valid, const uint8_t* key_valid, int64_t query_offset,
                      int B, int Sq, int Sk, int Hkv, int D, void* workspace, size_t workspace_bytes,
                      void* stream)
{
    g_last_error[0] = '\0';
    if (Hkv < 1) return fail(INKATTN_ERR_SHAPE, "Hkv=%d must be >= 1", Hkv);
    if (D != 64 && D != 128) return fail(INKATTN_ERR_UNSUPPORTED, "head_dim %d not built (64, 128)", D);
    MaskArgs ma;
    if (int rc = resolve_mask_args(valid, key_valid, nullptr, nullptr, query_offset, B, Sq, Sk, &ma)) return rc;
    if ((size_t)B * Sk == 0) return INKATTN_OK;
    if (!v) return fail(INKATTN_ERR_NULL, "v is NULL");
    if (!aligned(v, 16)) return fail(INKATTN_ERR_ALIGN, "v must be 16-byte aligned");
    if (int rc = check_tile_counts(B, Sq, Sk, Hkv, Hkv)) return rc;
    if (int rc = check_workspace(workspace, workspace_bytes, fwd_workspace_bytes(B, Sq, Sk, Hkv, D))) return rc;
    return launch_stage((const __bf16*)v, ma.key_valid, B, Sq, Sk, Hkv, D, (long long)Sk * Hkv * D, (long long)Hkv * D,
                        D, workspace, (hipStream_t)stream);
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
    if (int rc = check_fwd_args(q, k, v, profiles, profiles_dtype, sink, B, Sq, Sk, Hq, Hkv, D, E, out, lse))
        return rc;
    MaskArgs ma;
    if (int rc = resolve_mask_args(valid, key_valid, positions, key_positions, query_offset, B, Sq, Sk, &ma))
        return rc;
    if (window >= (int64_t(1) << 31) || window < 0) window = 0;
    if ((size_t)B * Sq == 0) return INKATTN_OK;   // nothing to write
    if ((size_t)Sk * Hkv * D * 2 >= (size_t(1) << 32))
        return fail(INKATTN_ERR_SHAPE, "one batch row of k / v must stay below 4 GiB");
    if (int rc = check_tile_counts(B, Sq, Sk, Hq, Hkv)) return rc;
    if (int rc = check_workspace(workspace, workspace_bytes, fwd_workspace_bytes(B, Sq, Sk, Hkv, D))) return rc;

    const long long sq_h = (long long)Hq * D, sk_h = (long long)Hkv * D;
    return run_forward(q, k, workspace, profiles, profiles_dtype, sink, valid, ma, positions, (int)window,
                       (int)query_offset, B, Sq, Sk, Hq, Hkv, D, E, out, 0, lse,
                       Strides{Sq * sq_h, sq_h, D}, Strides{Sk * sk_h, sk_h, D}, Strides{Sq * sq_h, sq_h, D},
                       Strides{(long long)Sq * Hq, Hq, 1}, Strides{(long long)Sq * Hq, Hq, 1},
                       (float)(1.0 / std::sqrt((double)D) * 1.4426950408889634), (hipStream_t)stream);
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
    if (int rc = check_fwd_args(q, k, v, profiles, profiles_dtype, sink, B, Sq, Sk, Hq, Hkv, D, E, out, lse))
        return rc;
    MaskArgs ma;
    if (int rc = resolve_mask_args(valid, key_valid, positions, key_positions, query_offset, B, Sq, Sk, &ma))
        return rc;
    if ((size_t)B * Sq == 0) return INKATTN_OK;
    if ((size_t)Sk * Hkv * D * 2 >= (size_t(1) << 32))
        return fail(INKATTN_ERR_SHAPE, "one batch row of k / v must stay below 4 GiB");
    if (int rc = check_tile_counts(B, Sq, Sk, Hq, Hkv)) return rc;
    if (int rc = check_workspace(workspace, workspace_bytes, fwd_workspace_bytes(B, Sq, Sk, Hkv, D))) return rc;
    if (int rc = attn_plan(valid, key_valid, positions, key_positions, query_offset, B, Sq, Sk, workspace,
                           workspace_bytes, stream))
        return rc;
    if (int rc = attn_stage_values(v, valid, key_valid, query_offset, B, Sq, Sk, Hkv, D, workspace,
                                   workspace_bytes, stream))
        return rc;
    return attn_fwd_planned(q, k, v, profiles, profiles_dtype, sink, valid, key_valid, positions, key_positions,
                            window, query_offset, B, Sq, Sk, Hq, Hkv, D, E, out, lse, workspace, workspace_bytes,
                            stream);
}

int attn_fwd_relproj(const void* q, const void* k, const void* v,
                     const void* rfeat, const void* table, int table_heads, int d_rel,
                     const float* sink, const uint8_t* valid, const uint8_t* key_valid,
                     const int32_t* positions, const int32_t* key_positions,
                     int64_t window, int64_t query_offset,
                     int B, int Sq, int Sk, int Hq, int Hkv, int D, int E,
                     float* out, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream)
{
    g_last_error[0] = '\0';
    if (d_rel != 16 && d_rel != 32)
        return fail(INKATTN_ERR_UNSUPPORTED, "relative feature width %d not built (16, 32)", d_rel);
    if (Hq >= 1 && table_heads != 1 && table_heads != Hq)
        return fail(INKATTN_ERR_SHAPE, "table_heads=%d must be 1 (shared) or Hq=%d", table_heads, Hq);
    // the profile checks of attn_fwd stand for the feature tensor (same rows, E entries per row)
    if (int rc = check_fwd_args(q, k, v, rfeat, INKATTN_BF16, sink, B, Sq, Sk, Hq, Hkv, D, E, out, lse)) return rc;
    if ((size_t)E * d_rel * 2 >= (size_t(1) << 32)) return fail(INKATTN_ERR_SHAPE, "table slice above 4 GiB");
    MaskArgs ma;
    if (int rc = resolve_mask_args(valid, key_valid, positions, key_positions, query_offset, B, Sq, Sk, &ma))
        return rc;
    if ((size_t)B * Sq == 0) return INKATTN_OK;
    if (!table) return fail(INKATTN_ERR_NULL, "table is NULL");
    if (!aligned(rfeat, 16) || !aligned(table, 16))
        return fail(INKATTN_ERR_ALIGN, "rfeat and table must be 16-byte aligned");
    if ((size_t)Sk * Hkv * D * 2 >= (size_t(1) << 32))
        return fail(INKATTN_ERR_SHAPE, "one batch row of k / v must stay below 4 GiB");
    if (window >= (int64_t(1) << 31) || window < 0) window = 0;
    if (int rc = check_tile_counts(B, Sq, Sk, Hq, Hkv)) return rc;
    if (int rc = check_workspace(workspace, workspace_bytes, fwd_workspace_bytes(B, Sq, Sk, Hkv, D))) return rc;
    if (int rc = attn_plan(valid, key_valid, positions, key_positions, query_offset, B, Sq, Sk, workspace,
                           workspace_bytes, stream))
        return rc;
    if (int rc = attn_stage_values(v, valid, key_valid, query_offset, B, Sq, Sk, Hkv, D, workspace,
                                   workspace_bytes, stream))
        return rc;
    RelArgs rel;
    rel.rfeat = rfeat;
    rel.table = table;
    rel.d_rel = d_rel;
    rel.r_bs = (long long)Sq * Hq * d_rel;
    rel.r_ts = (long long)Hq * d_rel;
    rel.r_hs = d_rel;
    rel.t_hs = table_heads == 1 ? 0 : (long long)E * d_rel;
    const long long sq_h = (long long)Hq * D, sk_h = (long long)Hkv * D;
    return run_forward(q, k, workspace, nullptr, INKATTN_F32, sink, valid, ma, positions, (int)window,
                       (int)query_offset, B, Sq, Sk, Hq, Hkv, D, E, out, 0, lse,
                       Strides{Sq * sq_h, sq_h, D}, Strides{Sk * sk_h, sk_h, D}, Strides{Sq * sq_h, sq_h, D},
                       Strides{(long long)Sq * Hq, Hq, 1}, Strides{(long long)Sq * Hq, Hq, 1},
                       (float)(1.0 / std::sqrt((double)D) * 1.4426950408889634), (hipStream_t)stream, rel);
}

int attn_fwd_noalloc(const void* q, const void* k, const void* v,
                     const void* profiles, int profiles_dtype,
                     const float* sink, const uint8_t* valid, const uint8_t* key_valid,
                     const int32_t* positions, const int32_t* key_positions,
                     int64_t window, int64_t query_offset,
                     int B, int Sq, int Sk, int Hq, int Hkv, int D, int E,
                     float* out, float* lse, void* stream)
{
    g_last_error[0] = '\0';
    if (int rc = check_fwd_args(q, k, v, profiles, profiles_dtype, sink, B, Sq, Sk, Hq, Hkv, D, E, out, lse))
        return rc;
    MaskArgs ma;
    if (int rc = resolve_mask_args(valid, key_valid, positions, key_positions, query_offset, B, Sq, Sk, &ma))
        return rc;
    if ((size_t)B * Sq == 0) return INKATTN_OK;
    if ((size_t)Sk * Hkv * D * 2 >= (size_t(1) << 32))
        return fail(INKATTN_ERR_SHAPE, "one batch row of k / v must stay below 4 GiB");
    if (int rc = check_tile_counts(B, Sq, Sk, Hq, Hkv)) return rc;
    const size_t need = fwd_workspace_bytes(B, Sq, Sk, Hkv, D);
    if (need > (size_t)INKATTN_NOALLOC_SCRATCH_BYTES)
        return fail(INKATTN_ERR_WORKSPACE,
                    "these sizes need %zu bytes of workspace, above the %zu bytes of the no-allocation scratch "
                    "(use attn_fwd with a workspace of attn_fwd_workspace_size bytes)",
                    need, (size_t)INKATTN_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (int rc = scratch_address(&ws)) return rc;
    // every part of the workspace is rewritten by each forward before it is
    // read (summaries, key start columns, values, flags): nothing to clear
    return attn_fwd(q, k, v, profiles, profiles_dtype, sink, valid, key_valid, positions, key_positions, window,
                    query_offset, B, Sq, Sk, Hq, Hkv, D, E, out, lse, ws, (size_t)INKATTN_NOALLOC_SCRATCH_BYTES,
                    stream);
}

int attn_debug_counts(const uint8_t* valid, const uint8_t* key_valid,
                      const int32_t* positions, const int32_t* key_positions,
                      int64_t window, int64_t query_offset, int B, int Sq, int Sk,
                      int32_t* n_allowed, void* stream)
{
    g_last_error[0] = '\0';
    MaskArgs ma;
    if (int rc = resolve_mask_args(valid, key_valid, positions, key_positions, query_offset, B, Sq, Sk, &ma))
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

int attn_debug_mask(const uint8_t* valid, const uint8_t* key_valid,
                    const int32_t* positions, const int32_t* key_positions,
                    int64_t window, int64_t query_offset, int B, int Sq, int Sk,
                    uint8_t* mask, void* stream)
{
    g_last_error[0] = '\0';
    MaskArgs ma;
    if (int rc = resolve_mask_args(valid, key_valid, positions, key_positions, query_offset, B, Sq, Sk, &ma))
        return rc;
    if (window >= (int64_t(1) << 31) || window < 0) window = 0;
    const size_t n = (size_t)B * Sq * Sk;
    if (n == 0) return INKATTN_OK;
    if (n > (size_t(1) << 32)) return fail(INKATTN_ERR_SHAPE, "mask of %zu entries is above the 2^32 limit", n);
    if (!mask) return fail(INKATTN_ERR_NULL, "mask is NULL");
    hipLaunchKernelGGL(debug_mask_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                       valid, ma.key_valid, positions, ma.key_positions, (int)window, (int)query_offset, Sq, Sk, n,
                       mask);
    return check_launch("debug_mask_kernel");
}

int attn_check_values(const void* workspace, size_t workspace_bytes, int B, int Sq, int Sk, int Hkv, int D,
                      void* stream)
{
    g_last_error[0] = '\0';
    if (B < 0 || Sq < 0 || Sk < 0 || Hkv < 1) return fail(INKATTN_ERR_SHAPE, "bad sizes");
    if (D != 64 && D != 128) return fail(INKATTN_ERR_UNSUPPORTED, "head_dim %d not built (64, 128)", D);
    if (Sq >= (1 << 30) || Sk >= (1 << 30)) return fail(INKATTN_ERR_SHAPE, "Sq / Sk must be below 2^30");
    const size_t nflags = (size_t)B * Hkv * ceil_div(Sk, BN);
    if (nflags == 0) return INKATTN_OK;
    if (int rc = check_workspace((void*)workspace, workspace_bytes, fwd_workspace_bytes(B, Sq, Sk, Hkv, D)))
        return rc;
    hipStream_t st = (hipStream_t)stream;
    const uint8_t* flags = (const uint8_t*)workspace + summaries_bytes(B, Sq, Sk) + values_bytes(B, Sk, Hkv, D);
    uint8_t* host = (uint8_t*)malloc(nflags);
    if (!host) return fail(INKATTN_ERR_SHAPE, "no host memory for %zu flags", nflags);
    hipError_t e = hipMemcpyAsync(host, flags, nflags, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) {
        free(host);
        return fail(INKATTN_ERR_LAUNCH, "reading the value flags: %s", hipGetErrorString(e));
    }
    size_t first = nflags;
    for (size_t t = 0; t < nflags && first == nflags; ++t)
        if (host[t]) first = t;
    free(host);
    if (first < nflags) {
        const size_t nKT = (size_t)ceil_div(Sk, BN);
        return fail(INKATTN_ERR_RANGE,
                    "v holds a value outside +-65504 (or not finite) at a real key: batch row %zu, K/V head %zu, "
                    "keys %zu..%zu",
                    first / ((size_t)Hkv * nKT), (first / nKT) % Hkv, (first % nKT) * BN, (first % nKT) * BN + BN - 1);
    }
    return INKATTN_OK;
}

int attn_debug_tiles(const uint8_t* valid, const uint8_t* key_valid,
                     const int32_t* positions, const int32_t* key_positions,
                     int64_t window, int64_t query_offset, int B, int Sq, int Sk,
                     uint8_t* tile_class, void* workspace, size_t workspace_bytes,
                     void* stream)
{
    g_last_error[0] = '\0';
    MaskArgs ma;
    if (int rc = resolve_mask_args(valid, key_valid, positions, key_positions, query_offset, B, Sq, Sk, &ma))
        return rc;
    if (window >= (int64_t(1) << 31) || window < 0) window = 0;
    const int nQB = ceil_div(Sq, BM), nKT = ceil_div(Sk, BN);
    const size_t n = (size_t)B * nQB * nKT;
    if (n == 0) return INKATTN_OK;
    if (!tile_class) return fail(INKATTN_ERR_NULL, "tile_class is NULL");
    if (int rc = check_workspace(workspace, workspace_bytes, summaries_bytes(B, Sq, Sk))) return rc;
    if (n >= (size_t(1) << 40)) return fail(INKATTN_ERR_SHAPE, "too many tiles");
    hipStream_t st = (hipStream_t)stream;
    TileSummary* qsum = (TileSummary*)workspace;
    TileSummary* ksum = qsum + (size_t)B * nQB;
    if (int rc = launch_summaries(valid, positions, ma.key_valid, ma.key_positions, (int)query_offset,
                                  B, Sq, Sk, workspace, st))
        return rc;
    hipLaunchKernelGGL(debug_tiles_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, qsum, ksum,
                       (int)window, (int)query_offset, B, Sq, Sk, nQB, nKT, tile_class);
    return check_launch("debug_tiles_kernel");
}

}  // extern "C"
