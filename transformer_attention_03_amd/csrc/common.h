// common.h -- pieces shared by the forward (inkattn.hip) and backward
// (attn_bwd.hip) translation units of the library: tile sizes, vector types,
// the per-tile mask summaries and the predicate every kernel masks with, the
// staged-operand key order, and the host-side argument / workspace helpers
// (defined in inkattn.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <climits>
#include <cstddef>
#include <cstdint>

namespace inkattn __attribute__((visibility("hidden"))) {

constexpr int BM = 32;   // query tokens per wave (MFMA N)
constexpr int BN = 64;   // keys per K/V tile (two MFMA M-blocks of 32)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4_u __attribute__((ext_vector_type(4), aligned(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

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

enum : int { TILE_SKIP = 0, TILE_MASKED = 1, TILE_FULL = 2 };

// Class of (query block, key tile) from the two summaries and the column
// ranges.  qlo / qhi: global columns of the block's first / last existing
// query; j0: first key column of the tile; key_hi: last existing key column.
__device__ __forceinline__ int classify_tile(const TileSummary& qs, int qlo, int qhi, int qcount,
                                             const TileSummary& ks, int j0, int key_hi, int kcount,
                                             int window)
{
    if (qcount <= 0 || qs.nvalid == 0 || ks.nvalid == 0) return TILE_SKIP;
    if (j0 > qhi) return TILE_SKIP;                                 // causal
    if (ks.amax < qs.amin || ks.amin > qs.amax) return TILE_SKIP;   // no common document
    if (window > 0 && qlo - key_hi >= window) return TILE_SKIP;     // nearest pair outside the window
    const bool one_doc = qs.amin == qs.amax && ks.amin == ks.amax && qs.amin == ks.amin;
    const bool all_real = qs.nvalid == qcount && ks.nvalid == kcount && qcount == BM && kcount == BN;
    const bool causal_full = key_hi <= qlo;
    const bool window_full = window <= 0 || qhi - j0 < window;
    return (one_doc && all_real && causal_full && window_full) ? TILE_FULL : TILE_MASKED;
}

// A value the compiler may not look through (no constant is split off it and
// no two loads using such offsets are merged).  The empty asm only exists in
// the device pass; the host pass never generates kernel code.
__device__ __forceinline__ unsigned opaque(unsigned x)
{
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+v"(x));
#endif
    return x;
}

// A wave-uniform value the compiler may not look through (kept in a scalar
// register; values derived from it are recomputed where they are used).
__device__ __forceinline__ unsigned opaque_s(unsigned x)
{
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+s"(x));
#endif
    return x;
}

// An LDS address the compiler may not look through: derived addresses are
// recomputed where they are used instead of being held in registers.
__device__ __forceinline__ lds_char* opaque_lds(lds_char* x)
{
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+s"(x));
#endif
    return x;
}

// An empty use of a value in registers: its computation must happen before
// this point (the device pass only; the host pass never generates kernel code).
template <typename T>
__device__ __forceinline__ void pin(const T& x)
{
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" ::"v"(x));
#endif
}

// Staged value tiles.  The staging pass writes, per (batch row, K/V head,
// 64-key tile), V^T as D rows of 64 fp16 values (128 B), the keys of each
// 16-key step in the order the PV MFMA consumes them: slot 8 hh + t of a step
// holds key 8 (t / 4) + 4 hh + ((t % 4) ^ 3), the key order of the P^T
// operand taken from the S^T accumulator.  A lane then reads its 8 keys of a
// step as one 16-byte chunk.  In LDS the 16-byte chunk c of row d sits at
// chunk c ^ vt_swz(d), which spreads the 16 rows of one read phase over all
// 64 banks.
__host__ __device__ constexpr int vt_slot(int key)   // key within the tile -> slot
{
    return 16 * (key / 16) + 8 * ((key / 4) % 2) + 4 * ((key % 16) / 8) + ((key % 4) ^ 3);
}
__device__ __forceinline__ int vt_swz(int d) { return (d >> 1) & 7; }

// Buffer resource over nrec bytes from base (reads past nrec return 0,
// writes past it are dropped).  The address and size go through
// readfirstlane, so the resource is known to be wave-uniform.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, size_t nrec)
{
    const unsigned long long a = (unsigned long long)base;
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
    const unsigned n = __builtin_amdgcn_readfirstlane((unsigned)nrec);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(((unsigned long long)hi << 32) | lo), 0, n, 0x00020000);
}

// ---------------------------------------------------------------------------
// Host helpers (inkattn.hip)
// ---------------------------------------------------------------------------
// Clears the message attn_last_error returns (start of every entry point).
void clear_error();

// Records a message for attn_last_error and returns status.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
bool aligned(const void* ptr, size_t a);
inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
size_t round256(size_t x);
size_t tile_summary_bytes(int B, int Sq, int Sk);
size_t summaries_bytes(int B, int Sq, int Sk);
size_t values_bytes(int B, int Sk, int Hkv, int D);
// per (batch row, K/V head, key tile) one byte: the staging found a value fp16 cannot hold
size_t value_flags_bytes(int B, int Sk, int Hkv);
// whole forward workspace: summaries, fp16 values, value flags
size_t fwd_workspace_bytes(int B, int Sq, int Sk, int Hkv, int D);
// tile and grid counts every launch of a forward needs must fit its index types
int check_tile_counts(int B, int Sq, int Sk, int Hq, int Hkv);

struct MaskArgs {
    const uint8_t* key_valid;
    const int32_t* positions;
    const int32_t* key_positions;
};

int resolve_mask_args(const uint8_t* valid, const uint8_t* key_valid, const int32_t* positions,
                      const int32_t* key_positions, int64_t query_offset, int B, int Sq, int Sk,
                      MaskArgs* outa);
int check_launch(const char* what);
int check_workspace(void* workspace, size_t workspace_bytes, size_t need);
// Pre-pass: per-tile summaries and key start columns at the head of workspace.
int launch_summaries(const uint8_t* valid, const int32_t* positions, const uint8_t* key_valid,
                     const int32_t* key_positions, int qoff, int B, int Sq, int Sk,
                     void* workspace, hipStream_t st);

}  // namespace inkattn
