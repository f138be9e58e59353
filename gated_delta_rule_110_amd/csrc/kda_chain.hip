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
// The state's V columns evolve independently, so each 256-thread workgroup
// owns one (sequence, head, 32-column V block); the state slice (128 x 32
// fp32) lives in MFMA accumulators and is shared through LDS as fp16 each
// step.  The four V-block workgroups of a head are placed on the same XCD
// (same blockIdx % 8) so that they share the head's per-chunk operands in
// that XCD's L2.  The optional initial state seeds S and the final state is
// written after the last chunk; passing one call's final state as the next
// call's initial state continues a sequence, which is the multi-turn state
// carry the forward call exposes ("¿Qué es la atención Kimi Delta…",
// 7minutos.es).
#include "kda_common.h"

using namespace kda;

namespace {

constexpr int kThreads = 256;
constexpr int kVB = 32;              // value columns per workgroup
constexpr int kNVB = kV / kVB;       // workgroups per (sequence, head)
constexpr int kSPad = kK + 8;        // LDS row pitches (halves)
constexpr int kUPad = kChunk + 8;
constexpr int kOPad = kVB + 8;

struct __align__(16) ChainSmem {
    _Float16 sSt[kVB * kSPad];       // S^T in fp16, [v][channel]
    _Float16 sUt[kVB * kUPad];       // Ut^T in fp16, [v][token]
    uint16_t sO[kChunk * kOPad];     // output tile, bf16 [token][v]
};

struct StepOps {
    h8 A[2][4];    // rows of -W (waves 0,1) or Qg (waves 2,3): [row tile][k step]
    h4 U[2][2];    // waves 0,1: U tile in accumulator layout [row tile][col tile]
    h8 Aq[2][2];   // waves 2,3: A_qk rows [row tile][k step]
    h8 Kb[2][2];   // Kbar^T rows [row tile][k step]
    f4 g[2];       // exp(G_n) for the lane's state rows [row tile]
};

__device__ __forceinline__ void load_step(StepOps &o, const ChainArgs &a, int64_t ws, int w, int vb,
                                          int r16, int cg) {
    const _Float16 *rows = (w < 2 ? a.Wn + ws * kWnElems : a.Qg + ws * kQgElems);
    const int rbase = 32 * (w & 1);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            o.A[rt][ks] = *reinterpret_cast<const h8 *>(rows + (rbase + 16 * rt + r16) * kK + 32 * ks + 8 * cg);
    if (w < 2) {
        const _Float16 *ut = a.Ut + ws * kUtElems;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
                o.U[rt][ct] = *reinterpret_cast<const h4 *>(ut + (kVB * vb + 16 * ct + r16) * kChunk + rbase + 16 * rt + 4 * cg);
    } else {
        const _Float16 *aq = a.Aqk + ws * kAqkElems;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                o.Aq[rt][ks] = *reinterpret_cast<const h8 *>(aq + (rbase + 16 * rt + r16) * kChunk + 32 * ks + 8 * cg);
    }
    const _Float16 *kb = a.Kbt + ws * kKbtElems;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            o.Kb[rt][ks] = *reinterpret_cast<const h8 *>(kb + (32 * w + 16 * rt + r16) * kChunk + 32 * ks + 8 * cg);
    const float *gn = a.gn + ws * kGnElems;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) o.g[rt] = *reinterpret_cast<const f4 *>(gn + 32 * w + 16 * rt + 4 * cg);
}

__global__ __launch_bounds__(kThreads, 2) void kda_chain_kernel(ChainArgs a) {
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

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int r16 = lane & 15;
    const int cg = lane >> 4;

    // state fragment: S[c = 32 w + 16 rt + 4 cg + e][v = 32 vb + 16 ct + r16]
    f4 S[2][2];
    const int64_t sbase = (n * H + h) * (int64_t)kK * kV;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t idx = sbase + (int64_t)(32 * w + 16 * rt + 4 * cg + e) * kV + kVB * vb + 16 * ct + r16;
                float s = 0.f;
                if (a.h0) s = a.h0_bf16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(a.h0)[idx])
                                        : reinterpret_cast<const float *>(a.h0)[idx];
                S[rt][ct][e] = s;
            }

    StepOps cur, nxt;
    if (nchunks > 0) load_step(cur, a, c0 * H + h, w, vb, r16, cg);

    for (int64_t s = 0; s < nchunks; ++s) {
        if (s + 1 < nchunks) load_step(nxt, a, (c0 + s + 1) * H + h, w, vb, r16, cg);

        // (a) S -> LDS as fp16, transposed
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                h4 sv;
                sv[0] = (_Float16)S[rt][ct][0]; sv[1] = (_Float16)S[rt][ct][1];
                sv[2] = (_Float16)S[rt][ct][2]; sv[3] = (_Float16)S[rt][ct][3];
                *reinterpret_cast<h4 *>(&sm.sSt[(16 * ct + r16) * kSPad + 32 * w + 16 * rt + 4 * cg]) = sv;
            }
        lds_barrier();

        // (b) waves 0,1: Ut = U - W S (rows 32w..);  waves 2,3: Qg S (rows 32(w-2)..)
        f4 X[2][2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                if (w < 2) {
                    X[rt][ct][0] = (float)cur.U[rt][ct][0]; X[rt][ct][1] = (float)cur.U[rt][ct][1];
                    X[rt][ct][2] = (float)cur.U[rt][ct][2]; X[rt][ct][3] = (float)cur.U[rt][ct][3];
                } else {
                    X[rt][ct] = f4{0, 0, 0, 0};
                }
            }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const h8 bs = *reinterpret_cast<const h8 *>(&sm.sSt[(16 * ct + r16) * kSPad + 32 * ks + 8 * cg]);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) X[rt][ct] = mfma16x16x32_f16(cur.A[rt][ks], bs, X[rt][ct]);
            }
        }
        if (w < 2) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    h4 uv;
                    uv[0] = (_Float16)X[rt][ct][0]; uv[1] = (_Float16)X[rt][ct][1];
                    uv[2] = (_Float16)X[rt][ct][2]; uv[3] = (_Float16)X[rt][ct][3];
                    *reinterpret_cast<h4 *>(&sm.sUt[(16 * ct + r16) * kUPad + 32 * w + 16 * rt + 4 * cg]) = uv;
                }
        }
        lds_barrier();

        // (c) S <- Diag(exp(G_n)) S + Kbar^T Ut ;  (d) waves 2,3: O = scale (Qg S + A_qk Ut)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) S[rt][ct] = S[rt][ct] * cur.g[rt];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const h8 bu = *reinterpret_cast<const h8 *>(&sm.sUt[(16 * ct + r16) * kUPad + 32 * ks + 8 * cg]);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) S[rt][ct] = mfma16x16x32_f16(cur.Kb[rt][ks], bu, S[rt][ct]);
                if (w >= 2) {
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt) X[rt][ct] = mfma16x16x32_f16(cur.Aq[rt][ks], bu, X[rt][ct]);
                }
            }
        }
        if (w >= 2) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sm.sO[(32 * (w - 2) + 16 * rt + 4 * cg + e) * kOPad + 16 * ct + r16] =
                            f32_to_bf16_bits(a.scale * X[rt][ct][e]);
        }
        lds_barrier();

        // output rows of this chunk: 64 rows x 32 columns, 16 bytes per thread
        {
            const int orow = tid >> 2, part = tid & 3;
            const int64_t rem = seqlen - kChunk * s;
            if (orow < rem) {
                const int64_t tok = tseq + kChunk * s + orow;
                uint4 val = *reinterpret_cast<const uint4 *>(&sm.sO[orow * kOPad + 8 * part]);
                *reinterpret_cast<uint4 *>(a.out + (tok * H + h) * kV + kVB * vb + 8 * part) = val;
            }
        }
        if (s + 1 < nchunks) cur = nxt;
    }

    if (a.ht) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t idx = sbase + (int64_t)(32 * w + 16 * rt + 4 * cg + e) * kV + kVB * vb + 16 * ct + r16;
                    if (a.ht_bf16) reinterpret_cast<uint16_t *>(a.ht)[idx] = f32_to_bf16_bits(S[rt][ct][e]);
                    else reinterpret_cast<float *>(a.ht)[idx] = S[rt][ct][e];
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
