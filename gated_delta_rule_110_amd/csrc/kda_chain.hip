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
// (sequence, head, 16-column V block).  Its first wave runs the chain: the
// 128 x 16 fp32 state slice lives in eight MFMA accumulator tiles, and because
// the intermediates are stored in fragment order with a matching k
// permutation, a pair of accumulator tiles converted to fp16 is directly the B
// operand of the next product -- no LDS round trip sits on the serial path.
// The second wave computes the outputs from the fp16 state and pseudo-value
// fragments the chain wave hands over through a double-buffered LDS slot, one
// barrier per chunk.  Each wave prefetches the next chunk's operands into
// registers while it works on the current one.
//
// The eight V-block workgroups of a head are placed on one XCD (same
// blockIdx % 8), so the head's per-chunk operands are fetched from HBM once
// into that XCD's L2 and shared.  The optional initial state seeds S and the
// final state is written after the last chunk; passing one call's final state
// as the next call's initial state continues a sequence, which is the
// multi-turn state carry the forward call exposes ("¿Qué es la atención Kimi
// Delta…", 7minutos.es).
#include "kda_common.h"

using namespace kda;

namespace {

constexpr int kThreads = 192;        // wave 0: state chain, wave 1: outputs, wave 2: L2 prefetch
#ifndef KDA_CHAIN_AHEAD
#define KDA_CHAIN_AHEAD 8
#endif
constexpr int kAhead = KDA_CHAIN_AHEAD;  // chunks the prefetch wave runs ahead of the chain
constexpr int kRing = 8;                 // chunks between a prefetch load and its use
constexpr int kVB = 16;              // value columns per workgroup
constexpr int kNVB = kV / kVB;       // workgroups per (sequence, head)

struct __align__(16) ChainSmem {
    h8 sS[2][4][64];   // state as fp16 B fragments [slot][k-block][lane]
    h8 sU[2][2][64];   // pseudo-values as fp16 B fragments
};

struct ChainOps {      // the chain wave's operands for one chunk
    h8 W[4][4];        // -W  [row tile][k-block]
    h8 K[8][2];        // Kbar^T [channel tile][k-block]
    h4 U[4];           // U in accumulator layout [row tile]
};

struct OutOps {        // the output wave's operands for one chunk
    h8 Q[4][4];        // Qg  [row tile][k-block]
    h8 A[4][2];        // A_qk [row tile][k-block]
};

__device__ __forceinline__ void load_chain_ops(ChainOps &o, const ChainArgs &a, int64_t ws, int vb,
                                               int lane) {
    const h8 *W = reinterpret_cast<const h8 *>(a.Wf + ws * kWfElems) + lane;
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) o.W[it][kb] = W[(it * 4 + kb) * 64];
    const h8 *K = reinterpret_cast<const h8 *>(a.Kf + ws * kKfElems) + lane;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) o.K[ct][kb] = K[(ct * 2 + kb) * 64];
    const h4 *U = reinterpret_cast<const h4 *>(a.Uf + ws * kUfElems) + vb * 4 * 64 + lane;
#pragma unroll
    for (int it = 0; it < 4; ++it) o.U[it] = U[it * 64];
}

__device__ __forceinline__ void load_out_ops(OutOps &o, const ChainArgs &a, int64_t ws, int lane) {
    const h8 *Q = reinterpret_cast<const h8 *>(a.Qf + ws * kQfElems) + lane;
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) o.Q[it][kb] = Q[(it * 4 + kb) * 64];
    const h8 *A = reinterpret_cast<const h8 *>(a.Af + ws * kAfElems) + lane;
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) o.A[it][kb] = A[(it * 2 + kb) * 64];
}

// exp(G_n) for the lane's state rows S[16 ct + 4 g + e][.].
__device__ __forceinline__ void load_decay(f4 (&gd)[8], const float *gn, int lane) {
    const f4 *G = reinterpret_cast<const f4 *>(gn) + (lane >> 4);
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) gd[ct] = G[4 * ct];
}

// Load this workgroup's share of one chunk's operands so that they are in the
// XCD's L2 when the chain and output waves load them a few chunks later.  The
// eight V-block workgroups of a head split the head's cache lines (one dword
// per 128-byte line).  The values are consumed kRing chunks later (folded
// into a checksum that is only stored through a null sink pointer), so the
// wave waits for each load long after issuing it, and loads complete in order.
__device__ __forceinline__ void touch_lines(const ChainArgs &a, int64_t ws, int vb, int lane, uint32_t &t0,
                                            uint32_t &t1) {
    const char *wf = reinterpret_cast<const char *>(a.Wf + ws * kWfElems);
    const char *qf = reinterpret_cast<const char *>(a.Qf + ws * kQfElems);
    const char *kf = reinterpret_cast<const char *>(a.Kf + ws * kKfElems);
    const char *af = reinterpret_cast<const char *>(a.Af + ws * kAfElems);
    const char *uf = reinterpret_cast<const char *>(a.Uf + ws * kUfElems);
    const char *gn = reinterpret_cast<const char *>(a.gn + ws * kGnElems);
    const int l = lane;
    const char *p0;  // lines 0..63 of the share: W, Qg, Kbar, U
    if (l < 16) p0 = wf + (16 * vb + l) * 128;
    else if (l < 32) p0 = qf + (16 * vb + l - 16) * 128;
    else if (l < 48) p0 = kf + (16 * vb + l - 32) * 128;
    else p0 = uf + (16 * vb + l - 48) * 128;
    const char *p1;  // lines 64..72: A_qk and exp(G_n) (lanes >= 8 share one line)
    if (l < 8) p1 = af + (8 * vb + l) * 128;
    else p1 = gn + (vb & 3) * 128;
    t0 = *reinterpret_cast<const uint32_t *>(p0);
    t1 = *reinterpret_cast<const uint32_t *>(p1);
}

// Two accumulator tiles (rows 4g+e of tile 2p and of tile 2p+1) -> one fp16 B
// fragment of k-block p.
__device__ __forceinline__ h8 pack_frag(const f4 &t0, const f4 &t1) {
    h8 r;
    r[0] = (_Float16)t0[0]; r[1] = (_Float16)t0[1]; r[2] = (_Float16)t0[2]; r[3] = (_Float16)t0[3];
    r[4] = (_Float16)t1[0]; r[5] = (_Float16)t1[1]; r[6] = (_Float16)t1[2]; r[7] = (_Float16)t1[3];
    return r;
}

// One chunk of the state chain.  S[ct] holds S[16 ct + 4 g + e][16 vb + r].
__device__ __forceinline__ void chain_step(ChainSmem &sm, f4 (&S)[8], const ChainOps &op, const f4 (&gd)[8],
                                           int slot, int lane) {
    h8 Sb[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        Sb[kb] = pack_frag(S[2 * kb], S[2 * kb + 1]);
        sm.sS[slot][kb][lane] = Sb[kb];
    }
    // Ut = U - W S: X[it] holds Ut[16 it + 4 g + e][16 vb + r]
    f4 X[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        X[it][0] = (float)op.U[it][0]; X[it][1] = (float)op.U[it][1];
        X[it][2] = (float)op.U[it][2]; X[it][3] = (float)op.U[it][3];
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int it = 0; it < 4; ++it) X[it] = mfma16x16x32_f16(op.W[it][kb], Sb[kb], X[it]);
    h8 Ub[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        Ub[kb] = pack_frag(X[2 * kb], X[2 * kb + 1]);
        sm.sU[slot][kb][lane] = Ub[kb];
    }
    lds_barrier();
    // S <- Diag(exp(G_n)) S + Kbar^T Ut
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) S[ct] = S[ct] * gd[ct];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) S[ct] = mfma16x16x32_f16(op.K[ct][kb], Ub[kb], S[ct]);
}

// Outputs of one chunk, computed transposed so that each lane ends up with four
// consecutive value columns of one token: O^T = S^T Qg^T + Ut^T A_qk^T.
__device__ __forceinline__ void out_step(ChainSmem &sm, const OutOps &op, int slot, int lane, float scale,
                                         uint16_t *out_chunk, int64_t row_stride, int64_t rows) {
    lds_barrier();
    h8 Sb[4], Ub[2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) Sb[kb] = sm.sS[slot][kb][lane];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) Ub[kb] = sm.sU[slot][kb][lane];
    f4 O[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) O[it] = f4{0, 0, 0, 0};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int it = 0; it < 4; ++it) O[it] = mfma16x16x32_f16(Sb[kb], op.Q[it][kb], O[it]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int it = 0; it < 4; ++it) O[it] = mfma16x16x32_f16(Ub[kb], op.A[it][kb], O[it]);
    // lane (r, g) holds O[16 it + r][16 vb + 4 g + e]
    const int r = lane & 15;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int row = 16 * it + r;
        if (row < rows) {
            uint2 pk;
            pk.x = (uint32_t)f32_to_bf16_bits(scale * O[it][0]) | ((uint32_t)f32_to_bf16_bits(scale * O[it][1]) << 16);
            pk.y = (uint32_t)f32_to_bf16_bits(scale * O[it][2]) | ((uint32_t)f32_to_bf16_bits(scale * O[it][3]) << 16);
            *reinterpret_cast<uint2 *>(out_chunk + row * row_stride) = pk;
        }
    }
}

__global__ __launch_bounds__(kThreads, 1) void kda_chain_kernel(ChainArgs a) {
    __shared__ ChainSmem sm;

    const int64_t H = a.H;
    const int64_t NH = a.N * H;
    // blockIdx -> (chain, V block) with all V blocks of a chain on one XCD
    const int64_t x = blockIdx.x;
    const int64_t xcd = x & 7;
    const int64_t sx = x >> 3;
    const int vb = (int)(sx % kNVB);
    const int64_t chain = (sx / kNVB) * 8 + xcd;
    if (chain >= NH) return;
    const int64_t n = chain / H, h = chain - (chain / H) * H;

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

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int g = lane >> 4;

    if (wave == 0) {
        // ---- state chain ---------------------------------------------------
        f4 S[8];
        const int64_t sbase = (n * H + h) * (int64_t)kK * kV + kVB * vb + r;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t idx = sbase + (int64_t)(16 * ct + 4 * g + e) * kV;
                float s = 0.f;
                if (a.h0) s = a.h0_bf16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(a.h0)[idx])
                                        : reinterpret_cast<const float *>(a.h0)[idx];
                S[ct][e] = s;
            }
        // Per step: the decay vector of this chunk is loaded first, then the
        // next chunk's operands; loads complete in order, so waiting for the
        // decay vector never waits for the prefetch.  The prefetch is issued
        // on every step (the last step reloads its own chunk) so that the
        // compiler's wait counts never have to cover a path without it.
        ChainOps A, B;
        f4 gd[8];
        const int64_t last = nchunks - 1;
        if (nchunks > 0) load_chain_ops(A, a, c0 * H + h, vb, lane);
        for (int64_t s = 0; s < nchunks; s += 2) {
            load_decay(gd, a.gn + ((c0 + s) * H + h) * kGnElems, lane);
            __builtin_amdgcn_sched_barrier(0);
            load_chain_ops(B, a, (c0 + (s + 1 < last ? s + 1 : last)) * H + h, vb, lane);
            chain_step(sm, S, A, gd, 0, lane);
            if (s + 1 >= nchunks) break;
            load_decay(gd, a.gn + ((c0 + s + 1) * H + h) * kGnElems, lane);
            __builtin_amdgcn_sched_barrier(0);
            load_chain_ops(A, a, (c0 + (s + 2 < last ? s + 2 : last)) * H + h, vb, lane);
            chain_step(sm, S, B, gd, 1, lane);
        }
        if (a.ht) {
#pragma unroll
            for (int ct = 0; ct < 8; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t idx = sbase + (int64_t)(16 * ct + 4 * g + e) * kV;
                    if (a.ht_bf16) reinterpret_cast<uint16_t *>(a.ht)[idx] = f32_to_bf16_bits(S[ct][e]);
                    else reinterpret_cast<float *>(a.ht)[idx] = S[ct][e];
                }
        }
    } else if (wave == 2) {
        // ---- L2 prefetch: chunk s + kAhead while the others work on chunk s --
        // Virtual step u touches chunk u + 1; steps u >= kAhead - 1 coincide with
        // chain step s = u - kAhead + 1 and end at that step's barrier.
        uint32_t acc = 0, r0[kRing], r1[kRing];
#pragma unroll
        for (int j = 0; j < kRing; ++j) { r0[j] = 0u; r1[j] = 0u; }
        const int64_t nu = nchunks > 0 ? nchunks + kAhead - 1 : 0;
        for (int64_t ub = 0; ub < nu; ub += kRing) {
#pragma unroll
            for (int j = 0; j < kRing; ++j) {
                const int64_t u = ub + j;
                // past the end, the last chunk is touched again (harmless, keeps the loads unconditional)
                const int64_t c = u + 1 < nchunks ? u + 1 : nchunks - 1;
                acc ^= r0[j] ^ r1[j];
                touch_lines(a, (c0 + c) * H + h, vb, lane, r0[j], r1[j]);
                if (u >= kAhead - 1 && u < nu) lds_barrier();
            }
        }
#pragma unroll
        for (int j = 0; j < kRing; ++j) acc ^= r0[j] ^ r1[j];
        if (a.sink) a.sink[lane] = acc;
    } else {
        // ---- outputs -------------------------------------------------------
        const int64_t row_stride = H * kV;
        uint16_t *out0 = a.out + (tseq * H + h) * kV + kVB * vb + 4 * g;
        OutOps A, B;
        const int64_t last = nchunks - 1;
        if (nchunks > 0) load_out_ops(A, a, c0 * H + h, lane);
        for (int64_t s = 0; s < nchunks; s += 2) {
            load_out_ops(B, a, (c0 + (s + 1 < last ? s + 1 : last)) * H + h, lane);
            out_step(sm, A, 0, lane, a.scale, out0 + kChunk * s * row_stride, row_stride, seqlen - kChunk * s);
            if (s + 1 >= nchunks) break;
            load_out_ops(A, a, (c0 + (s + 2 < last ? s + 2 : last)) * H + h, lane);
            out_step(sm, B, 1, lane, a.scale, out0 + kChunk * (s + 1) * row_stride, row_stride,
                     seqlen - kChunk * (s + 1));
        }
    }
}

// Packed batches: first chunk slot of each sequence, off[n] = sum_{m<n} ceil(len_m / 64).
__global__ __launch_bounds__(1024) void kda_chunk_table_kernel(const int64_t *cu, int64_t N, int32_t *off) {
    __shared__ int64_t part[1024];
    __shared__ int64_t carry;
    const int tid = threadIdx.x;
    if (tid == 0) carry = 0;
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
        if (n < N) off[n] = (int32_t)(carry + part[tid] - cnt);
        __syncthreads();
        if (tid == 1023) carry += part[1023];
        __syncthreads();
    }
    if (tid == 0) off[N] = (int32_t)carry;
}

}  // namespace

hipError_t kda_launch_chain(const ChainArgs &a, hipStream_t s) {
    const int64_t NH = a.N * a.H;
    if (NH <= 0) return hipSuccess;
    const int64_t groups = (NH + 7) / 8;
    const int64_t blocks = groups * 8 * kNVB;
    hipLaunchKernelGGL(kda_chain_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t kda_launch_chunk_table(const int64_t *cu, int64_t N, int32_t *chunk_off, hipStream_t s) {
    hipLaunchKernelGGL(kda_chunk_table_kernel, dim3(1), dim3(1024), 0, s, cu, N, chunk_off);
    return hipGetLastError();
}
