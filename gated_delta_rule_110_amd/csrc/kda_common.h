// kda_common.h -- internal definitions shared by the libkda HIP sources.
// Not part of the public ABI (that is include/kda.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

namespace kda {

constexpr int kChunk = 64;   // tokens per chunk
constexpr int kK = 128;      // key / query head dim (the only one supported)
constexpr int kV = 128;      // value head dim (the only one supported)

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef short s8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

// Per (chunk slot, head) intermediates written by the intra-chunk kernel and
// read by the state-chain kernel, fp16 unless stated.  They are stored in
// MFMA fragment order: each 16-byte (or 8-byte) group is exactly what one lane
// of a 16x16x32 MFMA holds, so every load and store moves 1 KiB (512 B) of
// contiguous memory per wave instruction.
//
// Lane l of a wave is (r = l & 15, g = l >> 4).  The state S and the chunk's
// pseudo-values live in MFMA accumulators, where lane (r, g) of tile t holds
// rows 16 t + 4 g + e (e = 0..3) of column r.  A pair of accumulator tiles
// (2 p, 2 p + 1) is fed straight back as the B operand of the 32-deep k-block
// p, so inside a k-block the lane's eight k slots j = 0..7 stand for the rows
//   perm(p, g, j) = 32 p + 4 g + j          (j < 4)
//                   32 p + 16 + 4 g + j - 4  (j >= 4)
// and every A operand that meets such a B operand is stored with its k index
// permuted the same way.
//
//   Wf [4 it][4 kb][64 lane][8]  -W[16 it + r][perm(kb, g, j)]            (negated)
//   Qf [4 it][4 kb][64 lane][8]   Qg[16 it + r][perm(kb, g, j)],  Qg = gamma * qhat
//   Kf [8 ct][2 kb][64 lane][8]   Kbar[perm(kb, g, j)][16 ct + r], Kbar_j = exp(G_n - G_j) khat_j
//   Af [4 it][2 kb][64 lane][8]   A_qk[16 it + r][perm(kb, g, j)]
//   Uf [8 vb][4 it][64 lane][4]   U[16 it + 4 g + e][16 vb + r]
//   gn [128] fp32                 exp(G_n), the chunk's total per-channel decay
// with W = (I + A_kk)^-1 Diag(b) (gamma * Khat) and U = (I + A_kk)^-1 Diag(b) V.
constexpr int64_t kWfElems = kChunk * kK;
constexpr int64_t kQfElems = kChunk * kK;
constexpr int64_t kKfElems = kK * kChunk;
constexpr int64_t kAfElems = kChunk * kChunk;
constexpr int64_t kUfElems = kChunk * kV;
constexpr int64_t kGnElems = kK;

struct Geometry {
    int64_t B, T, H, N;
    int64_t nc_fixed;     // chunks per sequence when not packed
    int64_t slots;        // chunk slots (upper bound when packed)
    bool varlen;
    int64_t segs;         // segments each sequence's chunk chain is split into (1 = not split)
    int64_t segc;         // chunks per segment (the last one may hold fewer)
    bool fused;           // the pipelined forward (kda_fused.hip) runs the call
};

struct WorkspaceLayout {
    size_t off_chunk_off;  // int32 [N + 1] per-sequence first chunk slot (packed only)
    size_t off_seq_order;  // int32 [N] sequences in chain dispatch order, longest first (packed only)
    size_t off_Wf, off_Qf, off_Kf, off_Af, off_Uf, off_gn;
    // split chains only: the segments as packed sequences (int64 [B segs + 1]
    // token offsets, int32 [B segs + 1] first chunk slots), the affine map of
    // every segment (fp32 [B segs, H, K, K] linear part, [B segs, H, K, V]
    // offset) and the state entering every segment (fp32 [B segs, H, K, V])
    size_t off_seg_cu, off_seg_off, off_mapM, off_mapN, off_sin;
    // pipelined forward only: int32 [slots * H] chunk ready flags, an int32 error
    // word and uint64 [8] producer item counters
    size_t off_flags, off_error, off_counters;
    size_t total;
};

struct IntraArgs {
    const uint16_t *q, *k, *v, *g, *beta;
    const float *A_log, *dt_bias;
    float lower_bound;
    const int64_t *cu;          // packed: cumulative lengths, else nullptr
    const int32_t *chunk_off;   // packed: [N + 1] first chunk slot of each sequence
    int64_t T, H, N, nc_fixed;
    _Float16 *Wf, *Qf, *Kf, *Af, *Uf;
    float *gn;
    int heads_fast;             // grid (H, slots) rather than (slots, H); set by the launcher
    int64_t slot_base;          // first chunk slot of this launch; set by the launcher
    int64_t piece_cap;          // kda_desc_t::launch_piece (0: launch size by the default rule)
};

struct ChainArgs {
    const _Float16 *Wf, *Qf, *Kf, *Af, *Uf;
    const float *gn;
    const int64_t *cu;
    const int32_t *chunk_off;
    const int32_t *seq_order;  // packed: the order chains are dispatched in (longest first), or nullptr
    int64_t T, H, N, nc_fixed;
    float scale;
    const void *h0;      // initial state [N,H,K,V] or nullptr
    void *ht;            // final state [N,H,K,V] or nullptr
    int h0_bf16, ht_bf16;
    uint16_t *out;       // [B,T,H,V] bf16
    // Map mode (map_mode != 0): no outputs and no h0 / ht.  Every V-block
    // workgroup runs its columns twice, from S = 0 (result to mapN) and from
    // S = I with U taken as 0 (result to mapM), both fp32 [N,H,K,128]: the
    // offset and the linear part of the chain's affine map S -> M S + N.
    int map_mode;
    float *mapM, *mapN;
    // With hs set the chain stores the fp32 state entering every chunk,
    // hs[chunk slot * H + h][16-column block][ct][lane][e] = S[16 ct + 4 (lane / 16) + e]
    // [16 block + lane % 16] (the chain's register layout, 16 bytes per lane and
    // row tile); with out also set it writes the outputs
    // as well (a forward that keeps the states for its backward), else none
    // (the backward's own forward pass, which needs the states only).
    float *hs;
    int64_t chain_base;  // first chain (in dispatch order) of this launch; set by the launcher
    int64_t piece_cap;   // kda_desc_t::launch_piece (0: launch size by the default rule)
};

// The sequential pass over the segments of split chains: for batch row b and
// head h, S_0 = h0[b, h] (zeros when h0 is null) and, for s = 0 .. segs - 1,
// S_{s+1} = M_s S_s + N_s with (M_s, N_s) the map of segment s; S_s (s < segs)
// goes to sin, S_segs to ht.
// With reverse set it is the same pass for the gradient of the state, last
// segment first: D_segs = h0[b, h] (the gradient of the final state, or zeros)
// and D_s = M_s^T D_{s+1} + N_s, with N_s the reverse chain of segment s run
// from a zero gradient; D_{s+1} (s < segs) goes to sin[segment s], the
// gradient leaving it, and D_0 to ht, the gradient of the initial state.
struct ScanArgs {
    const float *mapM, *mapN;   // [B segs, H, K, K] / [B segs, H, K, V] fp32
    float *sin;                 // [B segs, H, K, V] fp32
    const void *h0;             // [B, H, K, V] or nullptr
    void *ht;                   // [B, H, K, V] or nullptr
    int h0_bf16, ht_bf16;
    int reverse;
    int64_t B, H, segs;
};

struct DecodeArgs {
    const uint16_t *q, *k, *v, *g, *beta;   // [N,H,K] / [N,H,V] / [N,H] bf16
    const float *A_log, *dt_bias;
    float lower_bound, scale;
    int64_t N, H;
    const void *h0;      // state in [N,H,K,V] or nullptr (zeros)
    void *ht;            // state out [N,H,K,V] or nullptr; may alias h0
    int h0_bf16, ht_bf16;
    uint16_t *out;       // [N,H,V] bf16
    int64_t unit_base;   // first (sequence, head) of this launch; set by the launcher
    int64_t piece_cap;   // kda_desc_t::launch_piece (0: launch size by the default rule)
};

// ---- small numeric helpers --------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (hardware conversion; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ void unpack_bf16x8(const uint4 &r, float *o) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = __uint_as_float(w[i] << 16);
        o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

// Split x into two bf16 values hi + lo (hi = RNE(x), lo = RNE(x - hi)), using
// the hardware fp32 -> bf16 conversion (round to nearest even).
__device__ __forceinline__ void split_bf16(float x, short &hi, short &lo) {
    const __bf16 h = (__bf16)x;
    const short hs = __builtin_bit_cast(short, h);
    const float r = x - __uint_as_float((uint32_t)(uint16_t)hs << 16);
    hi = hs;
    lo = __builtin_bit_cast(short, (__bf16)r);
}

// Hardware transcendental approximations (about 1 ulp on normal values).
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ __forceinline__ float fast_log(float x) { return __builtin_amdgcn_logf(x) * 0.6931471805599453f; }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float fast_rsqrt(float x) { return __builtin_amdgcn_rsqf(x); }

// log2 of the per-channel decay, log2e * max(lb, -exp(A_log) softplus(x)) with
// x = g + dt_bias, nA = -exp(A_log) and lb2 = lb log2e.  softplus(x) = log(1 + e^x)
// is taken in three ranges so that it keeps its relative precision everywhere:
//   e^x < 2^-6 : the series t - t^2/2 + t^3/3 (relative error below 1e-6; the
//                plain log(1 + t) would lose the low bits of t once 1 + t
//                rounds, and return 0 below x = -16.6);
//   x > 15     : x itself (the remainder log1p(e^-x) < 4e-7 is below fp32
//                resolution, and e^x would overflow above x = 88.7);
//   otherwise  : log2(1 + e^x) on the hardware log.
// x = +inf gives the clamp lb, x = -inf gives 0.
__device__ __forceinline__ float gate_log2(float x, float nA, float lb2) {
    constexpr float kL2e = 1.4426950408889634f;
    const float t = __builtin_amdgcn_exp2f(x * kL2e);
    const float series = t * (kL2e - t * (0.5f * kL2e - t * (kL2e / 3.0f)));
    float sp2 = __builtin_amdgcn_logf(1.0f + t);  // log2(1 + t)
    sp2 = t < 0.015625f ? series : sp2;
    sp2 = x > 15.0f ? x * kL2e : sp2;
    return fmaxf(lb2, nA * sp2);
}

// DPP lane moves within 16-lane rows.
__device__ __forceinline__ float dpp_row_shr(float x, float fill, int s) {
    // lanes whose source lies before the row start keep `fill`
    switch (s) {
        case 1: return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(x), 0x111, 0xf, 0xf, false));
        case 2: return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(x), 0x112, 0xf, 0xf, false));
        case 4: return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(x), 0x114, 0xf, 0xf, false));
        default: return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(x), 0x118, 0xf, 0xf, false));
    }
}
__device__ __forceinline__ float dpp_row_shr_zero(float x, int s) {
    // lanes whose source lies before the row start read 0 (bound_ctrl)
    switch (s) {
        case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, true));
        case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, true));
        case 4: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, true));
        default: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, true));
    }
}
__device__ __forceinline__ float dpp_row_bcast15(float x) {
    // every lane of a 16-lane row receives the row's lane 15
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x15F, 0xf, 0xf, false));
}

// Barrier that orders LDS traffic only: outstanding global loads (prefetches)
// stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ b8 as_b8(const s8 &s) { return __builtin_bit_cast(b8, s); }

__device__ __forceinline__ f4 mfma16x16x32_f16(const h8 &a, const h8 &b, const f4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma16x16x32_bf16(const s8 &a, const s8 &b, const f4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(a), as_b8(b), c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma16x16x16_f16(const h4 &a, const h4 &b, const f4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// LDS byte address of a __shared__ object (what M0 and the ds_* instructions take).
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)(p);
}

// Each lane copies 4 bytes from global memory at p to LDS at lds + 4 * lane
// (global_load_lds; M0 holds the LDS base, and the s_nop is the wait state an
// M0 write needs before such a copy).  Used to pull cache lines into L2 ahead
// of their use: the copy has no destination register, and it is issued
// through inline asm, so the compiler neither waits for it nor makes later
// LDS accesses wait for it.  Only this wave's younger loads complete after it
// (vector-memory loads complete in order).
__device__ __forceinline__ void lds_copy4(const void *p, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" :: "v"(p), "{m0}"(lds) : "memory");
}

// Resolve packed sequence index of a chunk slot: largest n with off[n] <= slot.
__device__ __forceinline__ int64_t seq_of_slot(const int32_t *off, int64_t N, int64_t slot) {
    int64_t lo = 0, hi = N;  // invariant: off[lo] <= slot < off[hi] (off[N] > slot)
    while (hi - lo > 1) {
        int64_t mid = (lo + hi) >> 1;
        if (off[mid] <= slot) lo = mid; else hi = mid;
    }
    return lo;
}

// Largest grid piece (chains, chunk slots or decode units) one launch may
// cover: `dflt`, or `cap` when the caller asked for a smaller one
// (kda_desc_t::launch_piece > 0).  The defaults keep every launch within 2^30
// work-items, so only very large batches take several launches; a cap makes
// small inputs take that path too, so that it can be tested.
inline int64_t launch_piece(int64_t dflt, int64_t cap) {
    return cap > 0 && cap < dflt ? cap : dflt;
}

}  // namespace kda

// Kernel launchers (defined in the .hip files).
hipError_t kda_launch_chunk_table(const int64_t *cu, int64_t N, int32_t *chunk_off, int32_t *seq_order,
                                  hipStream_t s);
hipError_t kda_launch_intra(const kda::IntraArgs &a, int64_t slots, hipStream_t s);
hipError_t kda_launch_chain(const kda::ChainArgs &a, hipStream_t s);
hipError_t kda_launch_seg_table(int64_t B, int64_t T, int64_t segs, int64_t segc, int64_t *cu, int32_t *off,
                                hipStream_t s);
hipError_t kda_launch_seg_scan(const kda::ScanArgs &a, hipStream_t s);
hipError_t kda_launch_decode(const kda::DecodeArgs &a, hipStream_t s);
// The pipelined forward (kda_fused.hip): whether it handles these shapes, and
// its launch (the flag clear and the fused producer / consumer grid).
bool kda_fused_applies(int64_t N, int64_t H, bool varlen);
hipError_t kda_launch_fused(const kda::IntraArgs &in, const kda::ChainArgs &ch, int32_t *flags, int32_t *error,
                            unsigned long long *counters, int64_t slots, hipStream_t s);
