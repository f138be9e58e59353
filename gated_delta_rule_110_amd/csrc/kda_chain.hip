// kda_chain.hip -- inter-chunk state propagation fused with the output (gfx950).
//
// Carries the K x V state of every (sequence, head) across its chunks, which
// is the only serial dependency of the chunk-parallel form.  With the chunk
// quantities W, U, Kbar, Qg, A_qk and exp(G_n) written by the intra-chunk
// kernel, one chunk step is (S = state entering the chunk):
//
//   Ut_c = U - W S                         (pseudo-values of the chunk)
//   O_c  = scale * (Qg S + A_qk Ut_c)      (outputs of the chunk's tokens)
//   S   <- Diag(exp(G_n)) S + Kbar^T Ut_c  (state leaving the chunk)
//
// The state's V columns evolve independently, so each workgroup owns one
// (sequence, head, 16-column V block), with four waves:
//
//   wave 0 (chain)  keeps the 128 x 16 fp32 state slice in eight MFMA
//                   accumulator tiles.  The intermediates are stored in
//                   fragment order with a k permutation matching the
//                   accumulator layout, so two accumulator tiles converted to
//                   fp16 are directly the B operand of the next product -- no
//                   LDS round trip sits on the serial path.  It reads -W,
//                   Kbar^T, its U block and exp(G_n) from a three-slot LDS ring.
//   wave 1 (output) computes O from the fp16 state and pseudo-value fragments
//                   the chain wave hands over through a double-buffered LDS
//                   slot, loading the chunk's Qg and A_qk into registers just
//                   before the barrier that hands the fragments over.
//   wave 2 (loader) copies each chunk's ring operands straight from global
//                   memory into the ring (global_load_lds, no registers),
//                   kSlots - 1 chunks ahead of the chain.
//   wave 3 (L2)     loads this workgroup's share of the head's cache lines
//                   kAhead chunks ahead of the chain into the XCD's L2.
//
// One barrier per chunk orders the LDS hand-overs.  Vector-memory loads
// complete in order within a wave, so each wave only waits for loads that are
// older than the ones it issues for later chunks, and every prefetch is
// unconditional (past the end the last chunk is reloaded) so that the
// compiler's wait counts never cover a path without it.
//
// What bounds a chunk step is the CU's vector-memory path: each workgroup
// moves about 59 KiB per chunk through it (every V block needs the head's
// whole W, Kbar, Qg and A_qk), which takes about 1.07 us at the rate one CU
// sustains, longer than the chain wave's own arithmetic.
//
// With more than 32 chains, kda_chain_x2_kernel gives each workgroup two
// 16-column blocks (two chain waves on one operand ring, two output waves with
// half of the output rows each), so the head's operands cross each CU's load
// path once per 32 columns; with fewer chains that would leave CUs idle.
//
// The V-block workgroups of a head are placed on one XCD (same blockIdx % 8),
// so the head's per-chunk operands come from HBM once into that XCD's L2.
// The optional initial state seeds S and the final state is written after
// the last chunk; passing one call's final state as the next call's initial
// state continues a sequence, which is the multi-turn state carry the forward
// call exposes ("¿Qué es la atención Kimi Delta…", 7minutos.es).
//
// kda_chain_map_kernel is the same chain without outputs, used to split long
// chains (kda_segment.hip): it gives every chain its affine map S -> M S + N.
// Its output waves are chain waves too: in each V-block workgroup, chain wave c
// carries block c's columns of N (from S = 0) and wave kCB + c those of M (from
// S = I with the chunks' U taken as zero), all reading the same operand ring.
// kda_chain_map_x2_kernel does so with two blocks per workgroup, under the
// same rule as the two-block chain kernel.
#include "kda_common.h"

using namespace kda;

namespace {

constexpr int kAhead = 3;                // chunks the L2 prefetch runs ahead of the chain (measured: 3 beats 2 and 4-16)
constexpr int kTouchInFlight = 32;       // L2 prefetch copies allowed in flight: a tighter bound
                                         // stalls this wave, and the barrier, on HBM latency
constexpr int kVB = 16;                  // value columns per chain wave
constexpr int kBlocks = kV / kVB;        // 16-column blocks per head
// Chains at which the two-block workgroup is used: when the one-block grid
// (8 workgroups per chain) would not fit the GPU in one round.
constexpr int64_t kOneRoundWorkgroups = 256;

// Workgroup shapes; kCB = 16-column blocks of the state per workgroup.
//   kCB = 1: waves [chain, output, loader, L2 prefetch].
//   kCB = 2: waves [chain 0, chain 1, output 0, output 1, loader, L2 prefetch].
// The chain waves share the operand ring, so the head's -W and Kbar^T cross
// the CU's load path once for 32 columns instead of once per 16.  Output
// wave o computes the row tiles [kOutTiles o, kOutTiles (o + 1)) of the
// chunk's outputs for every block of the workgroup, loading only those rows
// of Qg and A_qk into registers: the two output waves of a two-block
// workgroup together load Qg and A_qk once.
template <int kCB>
struct Shape {
    static constexpr int kWaves = 2 * kCB + 2;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kNVB = kBlocks / kCB;       // workgroups per (sequence, head)
    static constexpr int kSlots = 3;                 // operand ring slots (2 measured 4% slower)
    static constexpr int kLead = kSlots - 1;         // chunks the ring copies run ahead of the chain
    static constexpr int kRingFrags = 33 + 2 * kCB;  // -W 16, Kbar^T 16, U 2 per block, exp(G_n) 1
    static constexpr int kOutTiles = 4 / kCB;        // 16-row output tiles per output wave
};
static_assert(Shape<1>::kSlots >= 2 && Shape<2>::kRingFrags * (Shape<2>::kSlots - 2) <= 63,
              "vmcnt holds at most 63 outstanding loads: kRingFrags (slots - 2) must fit");

template <int kCB>
struct __align__(16) ChainSmem {
    // per slot: -W frags [it*4+kb] (0..15), Kbar^T frags [16 + ct*2+kb] (16..31), the
    // workgroup's U blocks (32 + 2 c .. 33 + 2 c, [it][lane] of 8 bytes), exp(G_n) (32 + 2 kCB, 128 floats)
    h8 ring[Shape<kCB>::kSlots][Shape<kCB>::kRingFrags][64];
    h8 sS[2][kCB][4][64];      // state as fp16 B fragments [slot][block][k-block][lane]
    h8 sU[2][kCB][2][64];      // pseudo-values as fp16 B fragments
    uint32_t dump[2][64];      // landing place of the L2 prefetch copies (never read)
};

struct OutOps {        // the output wave's operands for one chunk
    h8 Q[4][4];        // Qg  [row tile][k-block]
    h8 A[4][2];        // A_qk [row tile][k-block]; [0][1] and [1][1] are zero and never loaded
};

__device__ __forceinline__ int64_t clamp_chunk(int64_t s, int64_t last) { return s < last ? s : last; }

// Row tiles [kIt0, kIt0 + kNt) of one chunk's Qg and A_qk.
template <int kIt0, int kNt>
__device__ __forceinline__ void load_out_ops(OutOps &o, const ChainArgs &a, int64_t ws, int lane) {
    const h8 *Q = reinterpret_cast<const h8 *>(a.Qf + ws * kQfElems) + lane;
#pragma unroll
    for (int it = kIt0; it < kIt0 + kNt; ++it)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) o.Q[it][kb] = Q[(it * 4 + kb) * 64];
    const h8 *A = reinterpret_cast<const h8 *>(a.Af + ws * kAfElems) + lane;
#pragma unroll
    for (int it = kIt0; it < kIt0 + kNt; ++it)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            if (kb == 0 || it >= 2) o.A[it][kb] = A[(it * 2 + kb) * 64];  // A_qk[i][j] = 0 for j > i
}

__device__ __forceinline__ void dma16(const void *g, void *l) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)g,
                                     (__attribute__((address_space(3))) void *)l, 16, 0, 0);
}

// Copy one chunk's -W and Kbar^T fragments (32 KiB), the workgroup's U blocks
// (2 KiB each) and exp(G_n) (512 B) straight from global memory into ring slot
// `slot`: kRingFrags vector-memory instructions with no registers; each lane's
// 16 bytes land at fragment base + lane * 16, the fragment order of the buffers.
template <int kCB>
__device__ __forceinline__ void dma_ring(ChainSmem<kCB> &sm, const ChainArgs &a, int64_t ws, int vb, int slot,
                                         int lane) {
    const h8 *W = reinterpret_cast<const h8 *>(a.Wf + ws * kWfElems) + lane;
    const h8 *K = reinterpret_cast<const h8 *>(a.Kf + ws * kKfElems) + lane;
#pragma unroll
    for (int f = 0; f < 16; ++f) dma16(W + f * 64, &sm.ring[slot][f][0]);
#pragma unroll
    for (int f = 0; f < 16; ++f) dma16(K + f * 64, &sm.ring[slot][16 + f][0]);
    const h8 *U = reinterpret_cast<const h8 *>(a.Uf + ws * kUfElems + vb * kCB * 4 * 64 * 4) + lane;
#pragma unroll
    for (int f = 0; f < 2 * kCB; ++f) dma16(U + f * 64, &sm.ring[slot][32 + f][0]);
    if (lane < 32) {
        const h8 *G = reinterpret_cast<const h8 *>(a.gn + ws * kGnElems) + lane;
        dma16(G, &sm.ring[slot][32 + 2 * kCB][0]);
    }
}

// Load this workgroup's share of one chunk's operands so that they are in the
// XCD's L2 when the other waves load them a few chunks later.  The V-block
// workgroups of a head split the head's cache lines: copy j covers the share of
// 16-column block vb kCB + j (one dword per 128-byte line).  The loads copy
// into an LDS area nobody reads: no destination registers, so this wave never
// has to wait for one except to bound how many are in flight.  Map mode and
// save mode read no Qg and no A_qk (kNoOut), so those lanes repeat a line the
// wave already touches (one request per line and instruction).
template <int kCB, bool kNoOut>
__device__ __forceinline__ void touch_lines(ChainSmem<kCB> &sm, const ChainArgs &a, int64_t ws, int vb, int lane) {
    const char *wf = reinterpret_cast<const char *>(a.Wf + ws * kWfElems);
    const char *qf = reinterpret_cast<const char *>(a.Qf + ws * kQfElems);
    const char *kf = reinterpret_cast<const char *>(a.Kf + ws * kKfElems);
    const char *af = reinterpret_cast<const char *>(a.Af + ws * kAfElems);
    const char *uf = reinterpret_cast<const char *>(a.Uf + ws * kUfElems);
    const char *gn = reinterpret_cast<const char *>(a.gn + ws * kGnElems);
    const int l = lane;
#pragma unroll
    for (int j = 0; j < kCB; ++j) {
        const int b = vb * kCB + j;
        const char *p0;  // lines 0..63 of the share: W, Qg, Kbar, U
        if (l < 16) p0 = wf + (16 * b + l) * 128;
        else if (l < 32) p0 = kNoOut ? wf + (16 * b + l - 16) * 128 : qf + (16 * b + l - 16) * 128;
        else if (l < 48) p0 = kf + (16 * b + l - 32) * 128;
        else p0 = uf + (16 * b + l - 48) * 128;
        const char *p1;  // lines 64..72: A_qk and exp(G_n) (lanes >= 8 share one line)
        if (l < 8 && !kNoOut) p1 = af + (8 * b + l) * 128;
        else p1 = gn + (b & 3) * 128;
        lds_copy4(p0, lds_addr(&sm.dump[0][0]));
        lds_copy4(p1, lds_addr(&sm.dump[1][0]));
    }
}

// Two accumulator tiles (rows 4g+e of tile 2p and of tile 2p+1) -> one fp16 B
// fragment of k-block p.
__device__ __forceinline__ h8 pack_frag(const f4 &t0, const f4 &t1) {
    h8 r;
    r[0] = (_Float16)t0[0]; r[1] = (_Float16)t0[1]; r[2] = (_Float16)t0[2]; r[3] = (_Float16)t0[3];
    r[4] = (_Float16)t1[0]; r[5] = (_Float16)t1[1]; r[6] = (_Float16)t1[2]; r[7] = (_Float16)t1[3];
    return r;
}

// One chunk of the state chain for block c of the workgroup.  S[ct] holds
// S[16 ct + 4 g + e][16 (vb kCB + c) + r]; the chunk's -W and Kbar^T fragments
// are in ring slot `rs`.  With kNoU the chunk's U is taken as zero (the linear
// part of the chunk map); kHandOver writes the fp16 state and pseudo-values
// for the output wave.
template <int kCB, bool kNoU, bool kHandOver>
__device__ __forceinline__ void chain_step(ChainSmem<kCB> &sm, f4 (&S)[8], int rs, int slot, int c, int lane) {
    h8 W[16];
#pragma unroll
    for (int f = 0; f < 16; ++f) W[f] = sm.ring[rs][f][lane];
    h8 Sb[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        Sb[kb] = pack_frag(S[2 * kb], S[2 * kb + 1]);
        if (kHandOver) sm.sS[slot][c][kb][lane] = Sb[kb];
    }
    // Ut = U - W S: X[it] holds Ut[16 it + 4 g + e][16 (vb kCB + c) + r]
    f4 X[4];
    if (kNoU) {
#pragma unroll
        for (int it = 0; it < 4; ++it) X[it] = f4{0, 0, 0, 0};
    } else {
        const h4 *Ul = reinterpret_cast<const h4 *>(&sm.ring[rs][32 + 2 * c][0]) + lane;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const h4 u = Ul[it * 64];
            X[it][0] = (float)u[0]; X[it][1] = (float)u[1]; X[it][2] = (float)u[2]; X[it][3] = (float)u[3];
        }
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int it = 0; it < 4; ++it) X[it] = mfma16x16x32_f16(W[it * 4 + kb], Sb[kb], X[it]);
    h8 K[16];   // read while the products above drain
#pragma unroll
    for (int f = 0; f < 16; ++f) K[f] = sm.ring[rs][16 + f][lane];
    h8 Ub[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        Ub[kb] = pack_frag(X[2 * kb], X[2 * kb + 1]);
        if (kHandOver) sm.sU[slot][c][kb][lane] = Ub[kb];
    }
    // exp(G_n)[16 ct + 4 g .. + 3] for the lane's rows, read before the
    // barrier: once this wave passes it, the ring slot is free for the loader
    f4 Gd[8];
    const f4 *Gl = reinterpret_cast<const f4 *>(&sm.ring[rs][32 + 2 * kCB][0]) + (lane >> 4);
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) Gd[ct] = Gl[4 * ct];
    lds_barrier();
    // S <- Diag(exp(G_n)) S + Kbar^T Ut
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) S[ct] = S[ct] * Gd[ct];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) S[ct] = mfma16x16x32_f16(K[ct * 2 + kb], Ub[kb], S[ct]);
}

// Row tiles [kIt0, kIt0 + kNt) of one chunk's outputs for every block of the
// workgroup, computed transposed so that each lane ends up with four
// consecutive value columns of one token: O^T = S^T Qg^T + Ut^T A_qk^T.  The
// Qg / A_qk rows are already in `op`; the state and pseudo-value fragments of
// each block come from hand-over slot `slot` after the barrier.
template <int kCB, int kIt0, int kNt>
__device__ __forceinline__ void out_step(ChainSmem<kCB> &sm, const OutOps &op, int slot, int lane, float scale,
                                         uint16_t *out_chunk, int64_t row_stride, int64_t rows) {
    lds_barrier();
    const int r = lane & 15;
#pragma unroll
    for (int c = 0; c < kCB; ++c) {
        h8 Sb[4], Ub[2];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) Sb[kb] = sm.sS[slot][c][kb][lane];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) Ub[kb] = sm.sU[slot][c][kb][lane];
        f4 O[kNt];
#pragma unroll
        for (int j = 0; j < kNt; ++j) O[j] = f4{0, 0, 0, 0};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int j = 0; j < kNt; ++j) O[j] = mfma16x16x32_f16(Sb[kb], op.Q[kIt0 + j][kb], O[j]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < kNt; ++j)
                if (kb == 0 || kIt0 + j >= 2) O[j] = mfma16x16x32_f16(Ub[kb], op.A[kIt0 + j][kb], O[j]);
        // lane (r, g) holds O[16 it + r][16 (vb kCB + c) + 4 g + e]
#pragma unroll
        for (int j = 0; j < kNt; ++j) {
            const int row = 16 * (kIt0 + j) + r;
            if (row < rows) {
                uint2 pk;
                pk.x = (uint32_t)f32_to_bf16_bits(scale * O[j][0]) | ((uint32_t)f32_to_bf16_bits(scale * O[j][1]) << 16);
                pk.y = (uint32_t)f32_to_bf16_bits(scale * O[j][2]) | ((uint32_t)f32_to_bf16_bits(scale * O[j][3]) << 16);
                *reinterpret_cast<uint2 *>(out_chunk + row * row_stride + kVB * c) = pk;
            }
        }
    }
}

// The output wave of row tiles [kIt0, kIt0 + kNt).  Qg and A_qk of a chunk are
// loaded into registers just before the barrier that hands over its state and
// pseudo-value fragments: the per-CU load path is the bottleneck, and deeper
// register prefetch (two or three chunks ahead) only adds loads in flight
// (measured equal or slower).
template <int kCB, int kIt0, int kNt, typename WsOf>
__device__ __forceinline__ void out_wave(ChainSmem<kCB> &sm, const ChainArgs &a, WsOf wsof, int64_t nchunks,
                                         uint16_t *out0, int64_t row_stride, int64_t seqlen, int lane) {
    OutOps A;
    lds_barrier();
    for (int64_t s = 0; s < nchunks; ++s) {
        load_out_ops<kIt0, kNt>(A, a, wsof(s), lane);
        out_step<kCB, kIt0, kNt>(sm, A, (int)(s & 1), lane, a.scale, out0 + kChunk * s * row_stride, row_stride,
                                 seqlen - kChunk * s);
    }
}

// The chain kernel's body; kMap selects map mode (ChainArgs::map_mode), which
// is a kernel of its own so that the ordinary chain is compiled without it;
// kSave stores the state entering every chunk to ChainArgs::hs; without kOut
// it writes no outputs (the backward's forward pass, which needs the states
// only): its output waves only keep the barrier count, and its L2 prefetch,
// like map mode's, skips Qg and A_qk.  Both are kernels of their own.
template <bool kMap, int kCB, bool kSave = false, bool kOut = !kSave>
__device__ __forceinline__ void chain_body(ChainSmem<kCB> &sm, const ChainArgs &a) {
    using Sh = Shape<kCB>;

    const int64_t H = a.H;
    const int64_t NH = a.N * H;
    // blockIdx -> (chain, V-block workgroup) with all workgroups of a chain on one XCD
    const int64_t x = blockIdx.x;
    const int64_t xcd = x & 7;
    const int64_t sx = x >> 3;
    const int vb = (int)(sx % Sh::kNVB);
    const int64_t chain = a.chain_base + (sx / Sh::kNVB) * 8 + xcd;
    if (chain >= NH) return;
    // packed batches: the i-th sequence in dispatch order (longest first), so
    // that short chains fill the GPU around the long ones instead of a long
    // one starting last
    const int64_t i_seq = chain / H, h = chain - i_seq * H;
    const int64_t n = a.seq_order ? (int64_t)a.seq_order[i_seq] : i_seq;

    int64_t c0, nchunks, tseq, seqlen;
    if (a.cu) {
        c0 = a.chunk_off[n];
        nchunks = a.chunk_off[n + 1] - c0;
        tseq = a.cu[n];
        seqlen = a.cu[n + 1] - tseq;
    } else {
        c0 = n * a.nc_fixed;
        nchunks = a.nc_fixed;
        tseq = n * a.T;
        seqlen = a.T;
    }
    const int64_t last = nchunks - 1;
    auto wsof = [&](int64_t s) { return (c0 + clamp_chunk(s, last)) * H + h; };

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int g = lane >> 4;

    if (wave < kCB || (kMap && wave < 2 * kCB)) {
        // ---- state chain ---------------------------------------------------
        // (map mode: wave c carries block c's N from S = 0, wave kCB + c its M
        // from S = I with U = 0; all read the same ring)
        const bool linear_part = kMap && wave >= kCB;
        const int c = linear_part ? wave - kCB : wave;  // block of the workgroup
        const int col0 = kVB * (vb * kCB + c);      // first value column of the block
        f4 S[8];
        const int64_t sbase = (n * H + h) * (int64_t)kK * kV + col0 + r;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t idx = sbase + (int64_t)(16 * ct + 4 * g + e) * kV;
                float v = 0.f;
                if (kMap) v = (linear_part && 16 * ct + 4 * g + e == col0 + r) ? 1.f : 0.f;
                else if (a.h0) v = a.h0_bf16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(a.h0)[idx])
                                             : reinterpret_cast<const float *>(a.h0)[idx];
                S[ct][e] = v;
            }
        if (nchunks > 0) {
            lds_barrier();  // ring slot 0 written by the loader
            int rs = 0;     // ring slot of chunk s
            for (int64_t s = 0; s < nchunks; ++s) {
                if constexpr (kSave) {
                    // in this lane layout (lane (r, g) holds rows 16 ct + 4 g + e of column
                    // col0 + r): [16-column block][ct][lane][e], one 16-byte store per ct
                    // (the texture path's instruction rate bounds the step, not its bytes)
                    f4 *hs = reinterpret_cast<f4 *>(a.hs + wsof(s) * (int64_t)(kK * kV)) +
                             (col0 / kVB) * (8 * 64) + lane;
#pragma unroll
                    for (int ct = 0; ct < 8; ++ct) hs[ct * 64] = S[ct];
                }
                if (!kMap) chain_step<kCB, false, kOut>(sm, S, rs, (int)(s & 1), c, lane);
                else if (linear_part) chain_step<kCB, true, false>(sm, S, rs, (int)(s & 1), c, lane);
                else chain_step<kCB, false, false>(sm, S, rs, (int)(s & 1), c, lane);
                rs = rs + 1 == Sh::kSlots ? 0 : rs + 1;
            }
        }
        if (kMap) {
            float *dst = linear_part ? a.mapM : a.mapN;
#pragma unroll
            for (int ct = 0; ct < 8; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[sbase + (int64_t)(16 * ct + 4 * g + e) * kV] = S[ct][e];
        } else if (a.ht) {
#pragma unroll
            for (int ct = 0; ct < 8; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t idx = sbase + (int64_t)(16 * ct + 4 * g + e) * kV;
                    if (a.ht_bf16) reinterpret_cast<uint16_t *>(a.ht)[idx] = f32_to_bf16_bits(S[ct][e]);
                    else reinterpret_cast<float *>(a.ht)[idx] = S[ct][e];
                }
        }
    } else if (wave < 2 * kCB) {
        // ---- outputs: row tiles of every block of the workgroup -------------
        if constexpr (!kOut) {
            if (nchunks > 0) {  // no outputs: the prologue barrier and one per chunk
                lds_barrier();
                for (int64_t s = 0; s < nchunks; ++s) lds_barrier();
            }
        } else if (nchunks > 0) {
            const int64_t row_stride = H * kV;
            uint16_t *out0 = a.out + (tseq * H + h) * kV + kVB * (vb * kCB) + 4 * g;
            constexpr int kNt = Sh::kOutTiles;
            if constexpr (kCB == 1) {
                out_wave<kCB, 0, kNt>(sm, a, wsof, nchunks, out0, row_stride, seqlen, lane);
            } else {
                if (wave == kCB) out_wave<kCB, 0, kNt>(sm, a, wsof, nchunks, out0, row_stride, seqlen, lane);
                else out_wave<kCB, kNt, kNt>(sm, a, wsof, nchunks, out0, row_stride, seqlen, lane);
            }
        }
    } else if (wave == 2 * kCB) {
        // ---- loader: -W / Kbar^T / U / exp(G_n) into the LDS ring -----------
        // Chunk s sits in slot s % kSlots.  Iteration u (between barriers u - 1
        // and u) starts the copy of chunk u + kLead into slot (u - 1) % kSlots:
        // chunk u - 1, which used it last, was read by the chain waves before
        // barrier u - 1.  It then waits for the copy of chunk u + 1 so that
        // barrier u publishes it for chain step u + 1.  This wave issues no
        // other vector-memory loads, and they complete in order, so "at most
        // kRingFrags (kLead - 1) outstanding" means exactly that every copy of
        // chunks up to u + 1 has landed.
        constexpr int kWait = Sh::kRingFrags * (Sh::kLead - 1);
        if (nchunks > 0) {
#pragma unroll
            for (int j = 0; j < Sh::kLead; ++j) dma_ring<kCB>(sm, a, wsof(j), vb, j, lane);
            asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kWait) : "memory");
            lds_barrier();  // ring slot 0 visible to the chain waves
            for (int64_t s = 0; s < nchunks; s += Sh::kSlots) {
#pragma unroll
                for (int j = 0; j < Sh::kSlots; ++j) {
                    const int64_t u = s + j;  // s is a multiple of kSlots
                    dma_ring<kCB>(sm, a, wsof(u + Sh::kLead), vb, (j + Sh::kLead) % Sh::kSlots, lane);
                    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kWait) : "memory");
                    if (u < nchunks) lds_barrier();
                }
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
    } else {
        // ---- L2 prefetch: chunk s + kAhead while the others work on chunk s --
        // Virtual step u touches chunk u + 1; steps u >= kAhead - 1 coincide with
        // chain step u - kAhead + 1 and end at that step's barrier (after the
        // prologue barrier the other waves pass first).
        if (nchunks > 0) {
            const int64_t nu = nchunks + kAhead - 1;
            bool prologue_done = false;
            for (int64_t u = 0; u < nu; ++u) {
                touch_lines<kCB, kMap || !kOut>(sm, a, wsof(u + 1), vb, lane);
                asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kTouchInFlight) : "memory");
                if (u >= kAhead - 1) {
                    if (!prologue_done) { lds_barrier(); prologue_done = true; }
                    lds_barrier();
                }
            }
            if (!prologue_done) lds_barrier();
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
    }
}

__global__ __launch_bounds__(Shape<1>::kThreads, 1) void kda_chain_kernel(ChainArgs a) {
    __shared__ ChainSmem<1> sm;
    chain_body<false, 1>(sm, a);
}
__global__ __launch_bounds__(Shape<2>::kThreads, 1) void kda_chain_x2_kernel(ChainArgs a) {
    __shared__ ChainSmem<2> sm;
    chain_body<false, 2>(sm, a);
}
__global__ __launch_bounds__(Shape<1>::kThreads, 1) void kda_chain_save_kernel(ChainArgs a) {
    __shared__ ChainSmem<1> sm;
    chain_body<false, 1, true>(sm, a);
}
__global__ __launch_bounds__(Shape<2>::kThreads, 1) void kda_chain_save_x2_kernel(ChainArgs a) {
    __shared__ ChainSmem<2> sm;
    chain_body<false, 2, true>(sm, a);
}
__global__ __launch_bounds__(Shape<1>::kThreads, 1) void kda_chain_out_save_kernel(ChainArgs a) {
    __shared__ ChainSmem<1> sm;
    chain_body<false, 1, true, true>(sm, a);
}
__global__ __launch_bounds__(Shape<2>::kThreads, 1) void kda_chain_out_save_x2_kernel(ChainArgs a) {
    __shared__ ChainSmem<2> sm;
    chain_body<false, 2, true, true>(sm, a);
}
__global__ __launch_bounds__(Shape<1>::kThreads, 1) void kda_chain_map_kernel(ChainArgs a) {
    __shared__ ChainSmem<1> sm;
    chain_body<true, 1>(sm, a);
}
__global__ __launch_bounds__(Shape<2>::kThreads, 1) void kda_chain_map_x2_kernel(ChainArgs a) {
    __shared__ ChainSmem<2> sm;
    chain_body<true, 2>(sm, a);
}

// Packed batches: first chunk slot of each sequence, off[n] = sum_{m<n} ceil(len_m / 64),
// and the order the chain kernel dispatches the sequences in: by chunk count,
// longest first, to within a factor of two (buckets of floor(log2(chunks)),
// empty sequences last; the order inside a bucket is arbitrary).  Every chain
// is computed independently, so the order changes only the schedule.
__device__ __forceinline__ int chunk_bucket(int64_t cnt) {  // 31 - floor(log2(cnt)); 32 when empty
    return cnt > 0 ? __clz((int)cnt) : 32;
}

__global__ __launch_bounds__(1024) void kda_chunk_table_kernel(const int64_t *cu, int64_t N, int32_t *off,
                                                               int32_t *order) {
    __shared__ int64_t part[1024];
    __shared__ int64_t carry;
    __shared__ int32_t bcount[33];  // sequences per bucket, then the next free position of each
    const int tid = threadIdx.x;
    if (tid == 0) carry = 0;
    if (tid < 33) bcount[tid] = 0;
    __syncthreads();
    for (int64_t base = 0; base < N; base += 1024) {
        const int64_t n = base + tid;
        int64_t cnt = 0;
        if (n < N) {
            const int64_t len = cu[n + 1] - cu[n];
            cnt = len > 0 ? (len + kChunk - 1) / kChunk : 0;
        }
        part[tid] = cnt;
        __syncthreads();
        for (int d = 1; d < 1024; d <<= 1) {  // inclusive Hillis-Steele scan
            const int64_t t = tid >= d ? part[tid - d] : 0;
            __syncthreads();
            part[tid] += t;
            __syncthreads();
        }
        if (n < N) {
            off[n] = (int32_t)(carry + part[tid] - cnt);
            atomicAdd(&bcount[chunk_bucket(cnt)], 1);
        }
        __syncthreads();
        if (tid == 1023) carry += part[1023];
        __syncthreads();
    }
    if (tid == 0) {
        off[N] = (int32_t)carry;
        int32_t start = 0;  // buckets in ascending order of 31 - log2: the longest first
        for (int b = 0; b <= 32; ++b) {
            const int32_t c = bcount[b];
            bcount[b] = start;
            start += c;
        }
    }
    __syncthreads();
    for (int64_t base = 0; base < N; base += 1024) {
        const int64_t n = base + tid;
        if (n < N) {
            const int64_t len = cu[n + 1] - cu[n];
            const int64_t cnt = len > 0 ? (len + kChunk - 1) / kChunk : 0;
            order[atomicAdd(&bcount[chunk_bucket(cnt)], 1)] = (int32_t)n;
        }
    }
}

}  // namespace


// Chains per launch are capped so that a launch stays within 2^30 work-items
// (a dispatch's grid is counted in 32-bit work-items per dimension): 65536
// groups of 8 chains, at 8 x 256 or 4 x 384 threads per chain.  Bigger
// batches (over half a million (sequence, head) chains) take several launches.
constexpr int64_t kMaxGroupsPerLaunch = 65536;

hipError_t kda_launch_chain(const ChainArgs &a, hipStream_t s) {
    const int64_t NH = a.N * a.H;
    if (NH <= 0) return hipSuccess;
    const int64_t groups = (NH + 7) / 8;  // chains in groups of 8, one per XCD
    // two blocks per workgroup when one block per workgroup would not fit the GPU in one round
    const bool wide = NH * kBlocks > kOneRoundWorkgroups;
    const int64_t piece = launch_piece(kMaxGroupsPerLaunch, a.piece_cap);
    for (int64_t g0 = 0; g0 < groups; g0 += piece) {
        const int64_t ng = groups - g0 < piece ? groups - g0 : piece;
        ChainArgs b = a;
        b.chain_base = 8 * g0;
        if (a.map_mode && wide)
            hipLaunchKernelGGL(kda_chain_map_x2_kernel, dim3((unsigned)(ng * 8 * Shape<2>::kNVB)),
                               dim3(Shape<2>::kThreads), 0, s, b);
        else if (a.map_mode)
            hipLaunchKernelGGL(kda_chain_map_kernel, dim3((unsigned)(ng * 8 * Shape<1>::kNVB)),
                               dim3(Shape<1>::kThreads), 0, s, b);
        else if (a.hs && a.out && wide)
            hipLaunchKernelGGL(kda_chain_out_save_x2_kernel, dim3((unsigned)(ng * 8 * Shape<2>::kNVB)),
                               dim3(Shape<2>::kThreads), 0, s, b);
        else if (a.hs && a.out)
            hipLaunchKernelGGL(kda_chain_out_save_kernel, dim3((unsigned)(ng * 8 * Shape<1>::kNVB)),
                               dim3(Shape<1>::kThreads), 0, s, b);
        else if (a.hs && wide)
            hipLaunchKernelGGL(kda_chain_save_x2_kernel, dim3((unsigned)(ng * 8 * Shape<2>::kNVB)),
                               dim3(Shape<2>::kThreads), 0, s, b);
        else if (a.hs)
            hipLaunchKernelGGL(kda_chain_save_kernel, dim3((unsigned)(ng * 8 * Shape<1>::kNVB)),
                               dim3(Shape<1>::kThreads), 0, s, b);
        else if (wide)
            hipLaunchKernelGGL(kda_chain_x2_kernel, dim3((unsigned)(ng * 8 * Shape<2>::kNVB)),
                               dim3(Shape<2>::kThreads), 0, s, b);
        else
            hipLaunchKernelGGL(kda_chain_kernel, dim3((unsigned)(ng * 8 * Shape<1>::kNVB)),
                               dim3(Shape<1>::kThreads), 0, s, b);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t kda_launch_chunk_table(const int64_t *cu, int64_t N, int32_t *chunk_off, int32_t *seq_order,
                                  hipStream_t s) {
    hipLaunchKernelGGL(kda_chunk_table_kernel, dim3(1), dim3(1024), 0, s, cu, N, chunk_off, seq_order);
    return hipGetLastError();
}
