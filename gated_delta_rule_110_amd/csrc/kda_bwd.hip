// kda_bwd.hip -- the backward pass of the KDA chunked forward (gfx950).
//
// The pages' kernels are forward-only ("性能与注意事项", zuobiaodaohang.com
// FlashKDA page); this is the gradient of the same operation, in the chunked
// form of the forward.  For one (sequence, head), with chunk c entering with
// state S = h_c and leaving with S' (the forward: Ut = U - W S,
// O = scale (Qg S + A_qk Ut), S' = Diag(exp(G_n)) S + Kbar^T Ut):
//
//   1. the forward chain, storing h_c (kda_chain.hip, save mode);
//   2. kda_bwd_prep_kernel, per chunk: normalised q and k, b, the cumulative
//      log-decay G, the decayed key Gram M (strictly lower) and
//      T = (I + Diag(b) M)^-1, in fp32, and the reverse chain's operands
//      (Kbar, A_qk^T, -W^T, Qg^T in fp16, exp(G_n) in fp32) in one block;
//   3. kda_bwd_chain_kernel, per (sequence, head, 16 state columns), last
//      chunk first, with dS the gradient of the state leaving the chunk:
//        dUt = scale A_qk^T dO + Kbar dS
//        dS <- Diag(exp(G_n)) dS - W^T dUt + scale Qg^T dO
//      storing dh_c (= dS before the step) and dUt; the final dS is the
//      initial state's gradient.  The step is affine in dS with the
//      transpose of the forward step's linear part, so split chains run it per
//      segment: from a zero gradient (map mode: the offset of the segment's
//      reverse map), then, after a scan with the forward maps transposed
//      (kda_segment.hip), from the gradient leaving the segment;
//   4. kda_bwd_main_kernel, per chunk, independently: with Y = V - (gamma Khat) S,
//      Ut = T Diag(b) Y and Z = T^T dUt,
//        dv = Diag(b) Z,   dQg = scale dO S^T,   Zw = -Z S^T,   dKbar = Ut dS'^T,
//        dA_qk = scale dO Ut^T (j <= i),   dA_kk = -Z Ut^T (j < i),
//      then the decayed Gram matrices' gradients, the per-channel decays
//      (a reverse cumulative sum of dG within the chunk), the gate, the norms
//      and beta;
//   5. kda_bwd_params_kernel: dA_log and ddt_bias, summed over the chunks.
//
// The preparation kernel and the per-chunk gradient's Gram-gradient phase run
// their products on the fp32 matrix cores (v_mfma_f32_16x16x4_f32): lane (r, g)
// gives A[r][g] and B[g][r] of a 16x16x4 step and holds C[4 g + e][r], so an
// operand can be read element by element from any layout.  The per-chunk
// gradient's other products (against S, dS', Ut, T and dUt) run on bf16
// 16x16x32 MFMAs with each fp32 operand split into bf16 hi + lo (dO is bf16
// already): three products (two against dO), good to about 2^-16 relative, in
// the same C layout.  The reverse chain, whose steps are serial, runs the fp16
// 16x16x16 product with fp32 accumulation on its fp16 operand block.
//
// Decay factors exp(G_i - G_j) inside a chunk are split around a reference
// row of each 16-row block (row 16 w + 8): with the log-decay >= -5 both
// halves stay within exp(+-40) for the rows of the block, and rows of earlier
// blocks only ever meet a factor <= 1.
#include "kda_bwd_args.h"

using namespace kda;

namespace {

constexpr int kThreads = 256;
constexpr int64_t kMaxUnitsPerLaunch = int64_t(1) << 22;  // 2^30 work-items per launch
constexpr int64_t kMaxGroupsPerLaunch = 65536;            // chain groups of 8 (8 x 8 x 320 threads each)

__device__ __forceinline__ f4 mma(float a, float b, const f4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float sigmoid_fast(float x) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}
// softplus on the hardware exp / log, in the three ranges of the forward's gate
// (series below e^x = 2^-6, x itself above 15, log(1 + e^x) between)
__device__ __forceinline__ float softplus_fast(float x) {
    const float t = __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
    const float series = t * (1.0f - t * (0.5f - t * (1.0f / 3.0f)));
    float sp = __builtin_amdgcn_logf(1.0f + t) * 0.6931471805599453f;
    sp = t < 0.015625f ? series : sp;
    return x > 15.0f ? x : sp;
}

// Eight fp32 values split into bf16 hi + lo operands (hi + lo carries about 16 bits of
// the significand, so a product of two split operands, the lo * lo term dropped, is good to
// about 2^-16 relative).
__device__ __forceinline__ void split8r(const float *x, s8 &hi, s8 &lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        short h, l;
        split_bf16(x[e], h, l);
        hi[e] = h;
        lo[e] = l;
    }
}
// ... of eight consecutive fp32 values (16-byte aligned).
__device__ __forceinline__ void split8(const float *p, s8 &hi, s8 &lo) {
    const float4 x0 = *reinterpret_cast<const float4 *>(p);
    const float4 x1 = *reinterpret_cast<const float4 *>(p + 4);
    const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    split8r(x, hi, lo);
}

// Sum over the 16 lanes of a row group (lanes r = 0..15 with the same g).
__device__ __forceinline__ float sum16(float x) {
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 8);
    return x;
}
// Sum over the four row groups (lanes with the same r).
__device__ __forceinline__ float sum4g(float x) {
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

// Token rows of chunk slot `slot`: first row t0 on the flattened [B*T] axis and
// the valid count L (1..64); false for a slot past the last chunk of a packed batch.
__device__ __forceinline__ bool chunk_rows(const BwdArgs &a, int64_t slot, int64_t &t0, int &L) {
    if (a.cu) {
        const int64_t total = a.chunk_off[a.N];
        if (slot >= total) return false;
        const int64_t n = seq_of_slot(a.chunk_off, a.N, slot);
        const int64_t i = slot - a.chunk_off[n];
        t0 = a.cu[n] + kChunk * i;
        const int64_t rem = a.cu[n + 1] - t0;
        L = (int)(rem < kChunk ? rem : kChunk);
    } else {
        const int64_t n = slot / a.nc_fixed;
        const int64_t i = slot - n * a.nc_fixed;
        t0 = n * a.T + kChunk * i;
        const int64_t rem = a.T - kChunk * i;
        L = (int)(rem < kChunk ? rem : kChunk);
    }
    return true;
}

// ---- 2. per-chunk preparation ------------------------------------------------

// The reverse chain's operands of one (chunk, head), fp16, written by the
// preparation kernel in the layouts the chain reads them in (every part a
// whole number of KiB, so the chain copies it with 1 KiB global_load_lds
// instructions):
//   Kn  [64][128]   Kbar[i][d] = exp(G_n[d] - G_i[d]) khat_i[d]
//   AqT [64][64]    A_qk^T[j][i], A_qk[i][j] = sum_d qhat_i khat_j exp(G_i - G_j) (j <= i)
//   WT  [128][64]   -W^T[d][i], W = T Diag(b) (gamma * Khat)
//   QgT [128][64]   Qg^T[d][i], Qg = gamma * qhat
//   gn  [128] fp32  exp(G_n)
// Rows are unpadded, with their 8-byte units of four columns permuted by the
// row's low four bits (co_idx), so that the chain's reads of four columns from
// 16 consecutive rows meet 16 different pairs of LDS banks; padding the rows
// instead cost a tenth more copies per chunk step.
constexpr int kTkP = 72;  // row pitch of the chain's fp16 dO^T and dUt^T tiles in LDS
constexpr int kCoKn = 0;
constexpr int kCoAq = kCoKn + kChunk * kK * 2;      // 16384
constexpr int kCoW = kCoAq + kChunk * kChunk * 2;   // 24576
constexpr int kCoQ = kCoW + kK * kChunk * 2;        // 40960
constexpr int kCoGn = kCoQ + kK * kChunk * 2;       // 57344
constexpr int kCoBytes = kCoGn + kK * 4;            // 57856
static_assert(kCoGn % 1024 == 0 && kCoBytes == kBwdChainOperandBytes, "chain operand block layout");
// element (row, col) of an operand part of kCols fp16 columns (64 or 128)
template <int kCols>
__device__ __forceinline__ int co_idx(int row, int col) {
    return row * kCols + ((((col >> 2) ^ (row & 15)) << 2) | (col & 3));
}

// The preparation kernel holds 64 of the 128 channels of q-hat, k-hat and G in
// LDS at a time (two passes), so that two workgroups fit on a CU (71 KB each):
// its phases are chains of dependent steps, and a second workgroup fills the
// waits.  The Gram sums of the two passes accumulate in registers in the same
// k order as one pass would; T takes the place of the q-hat tile once the Gram
// is done, and W, which needs T, is formed for the second half straight away
// and for the first half from the k-hat and G its threads kept in registers.
// (Two workgroups per CU leave each lane 256 registers; round trips of the
// halves through global memory instead missed L2 and cost 7%.)
constexpr int kHC = 64;       // channels per pass
constexpr int kHP = kHC + 1;  // row pitch of the half-channel tiles
struct PrepSmem {
    union {
        float q[kChunk][kHP];  // qhat, the pass's channels (through the Gram)
        float T[kChunk][kHP];  // T = (I + Diag(b) M)^-1 (after it)
    } u;
    float k[kChunk][kHP];      // khat, the pass's channels
    float G[kChunk][kHP];      // per-channel log-decay, cumulated in place
    float M[kChunk][kChunk + 1];
    union {
        float P[4][16][17];    // one 16 x 16 block product per wave (T solve)
        float tot[4][kHC];     // row-segment totals (cumulative sum)
    } v;
    float b[kChunk];
};
static_assert(sizeof(PrepSmem) <= 80 * 1024, "two preparation workgroups per CU");

__global__ __launch_bounds__(kThreads, 2) void kda_bwd_prep_kernel(BwdArgs a) {
    __shared__ PrepSmem sm;
    const int64_t ws = a.unit_base + blockIdx.x;  // chunk slot * H + head
    const int64_t slot = ws / a.H, h = ws - slot * a.H;
    int64_t t0;
    int L;
    if (!chunk_rows(a, slot, t0, L)) return;
    const int64_t H = a.H;
    const int tid = threadIdx.x;
    unsigned char *co = a.co + ws * (int64_t)kCoBytes;
    _Float16 *Kn = reinterpret_cast<_Float16 *>(co + kCoKn);
    _Float16 *AqT = reinterpret_cast<_Float16 *>(co + kCoAq);
    _Float16 *WT = reinterpret_cast<_Float16 *>(co + kCoW);
    _Float16 *QgT = reinterpret_cast<_Float16 *>(co + kCoQ);
    float *gno = reinterpret_cast<float *>(co + kCoGn);
    float *Go = a.G + ws * (kChunk * kK);

    // rows, norms, b and the per-channel log-decay; a quarter row per thread.
    // qhat and khat go out as they are; the first pass's half goes to LDS, and
    // the threads holding the second half keep it in registers until then.
    const int row = tid >> 2, qt = tid & 3;
    float qv[32], kv[32], gv[32];
    {
        const bool valid = row < L;
        const int64_t base = ((t0 + (valid ? row : 0)) * H + h) * kK + 32 * qt;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            unpack_bf16x8(*reinterpret_cast<const uint4 *>(a.q + base + 8 * i), qv + 8 * i);
            unpack_bf16x8(*reinterpret_cast<const uint4 *>(a.k + base + 8 * i), kv + 8 * i);
            unpack_bf16x8(*reinterpret_cast<const uint4 *>(a.g + base + 8 * i), gv + 8 * i);
        }
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int e = 0; e < 32; ++e) { sq += qv[e] * qv[e]; sk += kv[e] * kv[e]; }
        sq += __shfl_xor(sq, 1); sq += __shfl_xor(sq, 2);
        sk += __shfl_xor(sk, 1); sk += __shfl_xor(sk, 2);
        const float rq = valid ? 1.0f / sqrtf(sq + 1e-6f) : 0.f;
        const float rk = valid ? 1.0f / sqrtf(sk + 1e-6f) : 0.f;
        const float nA = -expf(a.A_log[h]);
        float dtb[32];  // loaded together, kept in registers (not reloaded inside the loop below)
#pragma unroll
        for (int e = 0; e < 32; e += 4) {
            const float4 x = *reinterpret_cast<const float4 *>(a.dt_bias + h * kK + 32 * qt + e);
            dtb[e] = x.x; dtb[e + 1] = x.y; dtb[e + 2] = x.z; dtb[e + 3] = x.w;
        }
#pragma unroll
        for (int e = 0; e < 32; ++e) asm volatile("" : "+v"(dtb[e]));
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            qv[e] *= rq;
            kv[e] *= rk;
            // the gate of every row, then the selection: under a per-element branch on the row's
            // validity the 32 exp / log chains would run one after another
            float z = fmaxf(a.lower_bound, nA * softplus_fast(gv[e] + dtb[e]));
            asm volatile("" : "+v"(z));
            gv[e] = valid ? z : 0.f;
        }
        if (qt < 2) {
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                sm.u.q[row][32 * qt + e] = qv[e];
                sm.k[row][32 * qt + e] = kv[e];
                sm.G[row][32 * qt + e] = gv[e];
            }
        }
        if (qt == 0) {
            // rows past the end read row 0's beta (in bounds) and discard it
            const float bl = bf16_bits_to_f32(a.beta[(t0 + (valid ? row : 0)) * H + h]);
            const float b = valid ? sigmoid_fast(bl) : 0.f;
            sm.b[row] = b;
            a.rq[ws * kChunk + row] = rq;
            a.rk[ws * kChunk + row] = rk;
            a.bb[ws * kChunk + row] = b;
        }
    }

    const int w = tid >> 6, lane = tid & 63, r = lane & 15, gq = lane >> 4;
    // M[i][j] = sum_d khat_i khat_j exp(G_i - G_j) (j < i) and A_qk (qhat_i, j <= i), by 16 x 16
    // tiles (I, J), J <= I: pair p of the ten goes to wave p % 4, so that the waves get 3, 3, 2
    // and 2 tiles.  exp(G_i - G_j) = exp(G_i - ref) exp(ref - G_j), ref = G[16 I + 8].
    f4 accM[3], accA[3];
#pragma unroll
    for (int t = 0; t < 3; ++t) { accM[t] = f4{0, 0, 0, 0}; accA[t] = accM[t]; }

    for (int half = 0; half < 2; ++half) {
        const int c0 = kHC * half;  // first channel of the pass
        if (half == 1) {
            // the second half of qhat, khat and the log-decay, from the registers that hold it
            __syncthreads();
            if (qt >= 2) {
#pragma unroll
                for (int e = 0; e < 32; ++e) {
                    sm.u.q[row][32 * (qt - 2) + e] = qv[e];
                    sm.k[row][32 * (qt - 2) + e] = kv[e];
                    sm.G[row][32 * (qt - 2) + e] = gv[e];
                }
            }
        }
        __syncthreads();
        // G_i = sum_{t <= i} a_t per channel: thread (channel c, row segment sg) sums 16 rows,
        // then adds the totals of the segments above it
        {
            const int c = tid & (kHC - 1), sg = tid >> 6;
            float run = 0.f;
#pragma unroll
            for (int i = 16 * sg; i < 16 * sg + 16; ++i) {
                run += sm.G[i][c];
                sm.G[i][c] = run;
            }
            sm.v.tot[sg][c] = run;
            __syncthreads();
            float off = 0.f;
            for (int s2 = 0; s2 < sg; ++s2) off += sm.v.tot[s2][c];
            if (sg > 0) {
#pragma unroll
                for (int i = 16 * sg; i < 16 * sg + 16; ++i) sm.G[i][c] += off;
            }
        }
        __syncthreads();
        {
            // the cumulated log-decay, Kbar (natural), Qg^T (four rows per store), exp(G_n)
            const float *Gn = sm.G[L - 1];
            // four consecutive channels per thread and pass: one 16-byte G store, one
            // 8-byte Kbar store (four columns are one unit of co_idx's permutation)
            for (int idx = tid; idx < kChunk * kHC / 4; idx += kThreads) {
                const int i = idx / (kHC / 4), d = 4 * (idx % (kHC / 4));
                float4 gv;
                h4 kv;
                float *gp = &gv.x;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    gp[e] = sm.G[i][d + e];
                    kv[e] = (_Float16)(__expf(Gn[d + e] - gp[e]) * sm.k[i][d + e]);
                }
                *reinterpret_cast<float4 *>(Go + i * kK + c0 + d) = gv;
                *reinterpret_cast<h4 *>(Kn + co_idx<kK>(i, c0 + d)) = kv;
            }
            for (int idx = tid; idx < kHC * (kChunk / 4); idx += kThreads) {
                const int d = idx >> 4, i0 = 4 * (idx & 15);
                h4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (_Float16)(__expf(sm.G[i0 + e][d]) * sm.u.q[i0 + e][d]);
                *reinterpret_cast<h4 *>(QgT + co_idx<kChunk>(c0 + d, i0)) = v;
            }
            if (tid < kHC) gno[c0 + tid] = __expf(Gn[tid]);
            // the first half's cumulated log-decay stays with the threads that hold its khat, for W
            if (half == 0 && qt < 2) {
#pragma unroll
                for (int e = 0; e < 32; ++e) gv[e] = sm.G[row][32 * qt + e];
            }
        }
        // this pass's part of the Gram sums (k = 4 ks + gq over the pass's channels)
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            const int p = w + 4 * t;
            if (p >= 10) break;
            const int I = p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3;
            const int J = p - I * (I + 1) / 2;
#pragma unroll 8
            for (int ks = 0; ks < kHC / 4; ++ks) {
                const int d = 4 * ks + gq;
                const float ref = sm.G[16 * I + 8][d];
                const float fa = __expf(sm.G[16 * I + r][d] - ref);
                const float bv = sm.k[16 * J + r][d] * __expf(ref - sm.G[16 * J + r][d]);
                accM[t] = mma(sm.k[16 * I + r][d] * fa, bv, accM[t]);
                accA[t] = mma(sm.u.q[16 * I + r][d] * fa, bv, accA[t]);
            }
        }
        if (half == 1) break;
        // W needs T, so the first half's part of it waits for the reload below
    }
    __syncthreads();  // the Gram is done: the qhat tile becomes T
    {
        float *Mk = a.Mk + ws * (kChunk * kChunk);
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            const int p = w + 4 * t;
            if (p >= 10) break;
            const int I = p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3;
            const int J = p - I * (I + 1) / 2;
            h4 at;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * I + 4 * gq + e, j = 16 * J + r;
                const float m = j < i ? accM[t][e] : 0.f;
                sm.M[i][j] = m;
                Mk[i * kChunk + j] = m;
                at[e] = (_Float16)(j <= i ? accA[t][e] : 0.f);
            }
            // A_qk^T[16 J + r][16 I + 4 gq .. + 3]
            *reinterpret_cast<h4 *>(AqT + co_idx<kChunk>(16 * J + r, 16 * I + 4 * gq)) = at;
        }
        // the tiles above the diagonal blocks are zero
        for (int idx = tid; idx < kChunk * kChunk / 4; idx += kThreads) {  // four columns of one tile
            const int i = idx >> 4, j = 4 * (idx & 15);
            if ((j >> 4) > (i >> 4)) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sm.M[i][j + e] = 0.f;
                    AqT[co_idx<kChunk>(j + e, i)] = (_Float16)0.f;
                    sm.u.T[i][j + e] = 0.f;
                }
                *reinterpret_cast<float4 *>(Mk + i * kChunk + j) = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
    }
    __syncthreads();
    // T = (I + A)^-1, A = Diag(b) M strictly lower, by 16 x 16 blocks.  First each
    // wave inverts its diagonal block by forward substitution down the columns,
    // one column per lane and the block's strict lower triangle in registers, so
    // only one multiply-add per column is on the serial path.
    if (gq == 0) {
        const int j = r;
        const int i0 = 16 * w;
        float Lt[120];  // A[i0 + rr][i0 + cc], cc < rr, row rr at offset rr (rr - 1) / 2
#pragma unroll
        for (int rr = 1; rr < 16; ++rr)
#pragma unroll
            for (int cc = 0; cc < rr; ++cc) Lt[rr * (rr - 1) / 2 + cc] = sm.b[i0 + rr] * sm.M[i0 + rr][i0 + cc];
        float xv[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) xv[rr] = rr == j ? 1.f : 0.f;
#pragma unroll
        for (int cc = 0; cc < 15; ++cc)
#pragma unroll
            for (int rr = cc + 1; rr < 16; ++rr) xv[rr] -= Lt[rr * (rr - 1) / 2 + cc] * xv[cc];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) sm.u.T[i0 + rr][i0 + j] = xv[rr];
    }
    __syncthreads();
    // Then column block J = w (w < 3), down its block rows:
    //   T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ,   I = J + 1 .. 3
    if (w < 3) {
        const int J = w;
        for (int I = J + 1; I < 4; ++I) {
            f4 pr = f4{0, 0, 0, 0};
            for (int K = J; K < I; ++K) {
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const int kk = 16 * K + 4 * s4 + gq;
                    const float av = sm.b[16 * I + r] * sm.M[16 * I + r][kk];
                    pr = mma(av, sm.u.T[kk][16 * J + r], pr);
                }
            }
            // lane (r, gq) holds P[4 gq + e][r]; through LDS for the B operand of T_II P
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.v.P[w][4 * gq + e][r] = pr[e];
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // one wave: LDS accesses in order
            f4 t = f4{0, 0, 0, 0};
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
                t = mma(sm.u.T[16 * I + r][16 * I + 4 * s4 + gq], sm.v.P[w][4 * s4 + gq][r], t);
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.u.T[16 * I + 4 * gq + e][16 * J + r] = -t[e];
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
    }
    __syncthreads();
    {
        float *Tm = a.Tm + ws * (kChunk * kChunk);
        for (int idx = tid; idx < kChunk * kChunk / 4; idx += kThreads) {  // 16 bytes per store
            const int i = idx >> 4, j = 4 * (idx & 15);
            *reinterpret_cast<float4 *>(Tm + i * kChunk + j) =
                make_float4(sm.u.T[i][j], sm.u.T[i][j + 1], sm.u.T[i][j + 2], sm.u.T[i][j + 3]);
        }
    }
    // W = T Diag(b) (gamma * Khat), stored as -W^T; T[i][j] = 0 for j > i.  The second
    // half's channels are in LDS; then the first half's come back from registers.
    for (int half = 1; half >= 0; --half) {
        const int c0 = kHC * half;
        if (half == 0) {
            __syncthreads();
            if (qt < 2) {
#pragma unroll
                for (int e = 0; e < 32; ++e) {
                    sm.k[row][32 * qt + e] = kv[e];
                    sm.G[row][32 * qt + e] = gv[e];
                }
            }
            __syncthreads();
        }
        f4 acc[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[ct] = f4{0, 0, 0, 0};
        for (int ks = 0; ks < 4 * (w + 1); ++ks) {
            const int j = 4 * ks + gq;
            const float av = sm.u.T[16 * w + r][j];
            const float bj = sm.b[j];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const int d = 16 * ct + r;
                acc[ct] = mma(av, bj * __expf(sm.G[j][d]) * sm.k[j][d], acc[ct]);
            }
        }
        // lane holds W[16 w + 4 gq + e][c0 + 16 ct + r] -> -W^T[c0 + 16 ct + r][16 w + 4 gq .. + 3]
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            h4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (_Float16)(-acc[ct][e]);
            *reinterpret_cast<h4 *>(WT + co_idx<kChunk>(c0 + 16 * ct + r, 16 * w + 4 * gq)) = v;
        }
    }
}

// ---- 3. the reverse state chain ----------------------------------------------

constexpr int kChainWaves = 6;  // 4 compute waves, the loader, the L2 prefetch
constexpr int kChainAhead = 3;  // chunks the L2 prefetch runs ahead of the chain
constexpr int kTouchInFlight = 8;  // L2 prefetch loads allowed in flight (two per chunk)

struct __align__(16) BwdChainSmem {
    unsigned char ops[2][kCoBytes];   // one chunk's operand block per slot (layout above)
    _Float16 dOT[2][16][kTkP];        // dO^T of the block's 16 columns (fp16)
    f4 red[4][4][64];                 // partial dUt tiles [wave][row tile][lane]
    _Float16 dUT[16][kTkP];           // dUt^T of the block (fp16)
    uint32_t dump[64];                // landing place of the L2 prefetch copies (never read)
};

__device__ __forceinline__ void copy16(const void *g, void *l) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)g,
                                     (__attribute__((address_space(3))) void *)l, 16, 0, 0);
}

__device__ __forceinline__ h4 pack_h4(const f4 &x) {
    h4 r;
    r[0] = (_Float16)x[0]; r[1] = (_Float16)x[1]; r[2] = (_Float16)x[2]; r[3] = (_Float16)x[3];
    return r;
}

__global__ __launch_bounds__(64 * kChainWaves, 1) void kda_bwd_chain_kernel(BwdArgs a) {
    __shared__ BwdChainSmem sm;
    const int64_t H = a.H;
    const int64_t NH = a.N * H;
    const int64_t x = blockIdx.x;
    const int64_t xcd = x & 7;
    const int64_t sx = x >> 3;
    const int vb = (int)(sx & 7);
    const int64_t chain = a.chain_base + (sx >> 3) * 8 + xcd;  // the 8 blocks of a chain on one XCD
    if (chain >= NH) return;
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
    const int col0 = 16 * vb;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;

    if (wave == 5) {
        // ---- L2 prefetch: this block's eighth of the operand lines of chunk
        // step s + kChainAhead, while the others work on step s (no destination
        // registers: the copies land in an LDS area nobody reads) ----------------
        if (nchunks > 0) {
            const int line = vb + 8 * lane;  // 500 lines of 128 B per chunk; lanes past the end repeat line vb
            const int64_t off = 128 * (int64_t)(line < kCoBytes / 128 ? line : vb);
            for (int64_t s = -1; s < nchunks; ++s) {
                const int64_t u = s + kChainAhead;
                const int64_t ci = nchunks - 1 - (u < nchunks ? u : nchunks - 1);
                lds_copy4(a.co + ((c0 + ci) * H + h) * (int64_t)kCoBytes + off, lds_addr(&sm.dump[0]));
                // and the chunk's dO rows of this block (one 32-byte piece per token row)
                const int64_t rows = seqlen - kChunk * ci;
                const int64_t tok = tseq + kChunk * ci + (lane < rows ? lane : 0);
                lds_copy4(a.dout + (tok * H + h) * kV + col0, lds_addr(&sm.dump[0]));
                asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kTouchInFlight) : "memory");
                lds_barrier();
                if (s >= 0) {
                    lds_barrier();
                    lds_barrier();
                }
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        return;
    }
    if (wave == 4) {
        // ---- loader: chunk ci into slot s.  The dO rows are loaded into registers
        // first, then the operand block is copied straight into LDS; dO^T is built
        // (bf16 -> fp16) after the step's second barrier, and the copies are waited
        // for only before its last one, so that neither is on the path of the
        // compute waves' first two barriers.  (Issuing the 57 copies takes most of
        // a step, the per-CU load path being the limit: splitting them over two
        // loader waves, more in flight, measured 12% slower.) ----------------------
        auto issue = [&](int64_t ci, int s, uint4 &p0, uint4 &p1) {
            const int64_t rows = seqlen - kChunk * ci;
            p0 = make_uint4(0, 0, 0, 0);
            p1 = p0;
            if (lane < rows) {
                const uint4 *p = reinterpret_cast<const uint4 *>(a.dout + ((tseq + kChunk * ci + lane) * H + h) * kV + col0);
                p0 = p[0];
                p1 = p[1];
            }
            const int64_t ws = (c0 + ci) * H + h;
            const unsigned char *src = a.co + ws * (int64_t)kCoBytes + 16 * lane;
#pragma unroll 4
            for (int f = 0; f < kCoGn / 1024; ++f) copy16(src + 1024 * f, &sm.ops[s][1024 * f]);
            if (lane < 32) copy16(src + kCoGn, &sm.ops[s][kCoGn]);
        };
        // dO^T: lane = token row (zero past the end)
        auto finish = [&](int s, const uint4 &p0, const uint4 &p1) {
            float f[16];
            unpack_bf16x8(p0, f);
            unpack_bf16x8(p1, f + 8);
#pragma unroll
            for (int c = 0; c < 16; ++c) sm.dOT[s][c][lane] = (_Float16)f[c];
        };
        if (nchunks > 0) {
            uint4 p0, p1;
            issue(nchunks - 1, 0, p0, p1);
            finish(0, p0, p1);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            lds_barrier();
            for (int64_t s = 0; s < nchunks; ++s) {
                const bool more = s + 1 < nchunks;
                const int nslot = (int)((s + 1) & 1);
                if (more) issue(nchunks - 2 - s, nslot, p0, p1);
                lds_barrier();
                lds_barrier();
                if (more) finish(nslot, p0, p1);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                lds_barrier();
            }
        }
        return;
    }

    // ---- compute waves: wave w carries state rows 32 w .. 32 w + 31 ----------
    const int w = wave;
    f4 dS[2];  // tile t: rows 16 (2 w + t) + 4 g + e, column col0 + r
    {
        const int64_t sb = (n * H + h) * (int64_t)(kK * kV) + col0 + r;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t idx = sb + (int64_t)(16 * (2 * w + t) + 4 * g + e) * kV;
                float v = 0.f;
                if (a.dht) v = a.dht_bf16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(a.dht)[idx])
                                          : reinterpret_cast<const float *>(a.dht)[idx];
                dS[t][e] = v;
            }
    }
    if (nchunks > 0) {
        lds_barrier();
        for (int64_t s = 0; s < nchunks; ++s) {
            const int64_t ci = nchunks - 1 - s;
            const int slot = (int)(s & 1);
            const int64_t ws = (c0 + ci) * H + h;
            const _Float16 *Kn = reinterpret_cast<const _Float16 *>(&sm.ops[slot][kCoKn]);
            const _Float16 *AqT = reinterpret_cast<const _Float16 *>(&sm.ops[slot][kCoAq]);
            const _Float16 *WT = reinterpret_cast<const _Float16 *>(&sm.ops[slot][kCoW]);
            const _Float16 *QgT = reinterpret_cast<const _Float16 *>(&sm.ops[slot][kCoQ]);
            const float *gn = reinterpret_cast<const float *>(&sm.ops[slot][kCoGn]);
            // the gradient of the state leaving this chunk
            if (!a.chain_map) {
                float *dh = a.dhs + ws * (int64_t)(kK * kV) + col0 + r;
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e) dh[(16 * (2 * w + t) + 4 * g + e) * kV] = dS[t][e];
            }
            // partial dUt over this wave's 32 state rows: Kbar[:, rows] dS[rows]; the B
            // operand of channel tile ct is the lane's own accumulator tile, in fp16
            f4 acc[4];
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) acc[jt] = f4{0, 0, 0, 0};
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int ct = 2 * w + t;
                const h4 bv = pack_h4(dS[t]);
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) {
                    const h4 av = *reinterpret_cast<const h4 *>(Kn + co_idx<kK>(16 * jt + r, 16 * ct + 4 * g));
                    acc[jt] = mfma16x16x16_f16(av, bv, acc[jt]);
                }
            }
            // scale A_qk^T dO for row tile w
            {
                f4 aq = f4{0, 0, 0, 0};
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const h4 av = *reinterpret_cast<const h4 *>(AqT + co_idx<kChunk>(16 * w + r, 16 * kb + 4 * g));
                    const h4 bv = *reinterpret_cast<const h4 *>(&sm.dOT[slot][r][16 * kb + 4 * g]);
                    aq = mfma16x16x16_f16(av, bv, aq);
                }
#pragma unroll
                for (int jt = 0; jt < 4; ++jt)
                    if (jt == w) acc[jt] += a.scale * aq;
            }
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) sm.red[w][jt][lane] = acc[jt];
            lds_barrier();
            // row tile w of dUt: lane holds dUt[16 w + 4 g + e][col0 + r]
            {
                const f4 u = sm.red[0][w][lane] + sm.red[1][w][lane] + sm.red[2][w][lane] + sm.red[3][w][lane];
                if (!a.chain_map) {
                    float *du = a.dUt + ws * (int64_t)(kChunk * kV) + col0 + r;
#pragma unroll
                    for (int e = 0; e < 4; ++e) du[(16 * w + 4 * g + e) * kV] = u[e];
                }
                *reinterpret_cast<h4 *>(&sm.dUT[r][16 * w + 4 * g]) = pack_h4(u);
            }
            lds_barrier();
            // dS <- Diag(exp(G_n)) dS - W^T dUt + scale Qg^T dO   (WT holds -W^T)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int ct = 2 * w + t;
                f4 nd, nq = f4{0, 0, 0, 0};
#pragma unroll
                for (int e = 0; e < 4; ++e) nd[e] = gn[16 * ct + 4 * g + e] * dS[t][e];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const h4 aw = *reinterpret_cast<const h4 *>(WT + co_idx<kChunk>(16 * ct + r, 16 * kb + 4 * g));
                    const h4 bu = *reinterpret_cast<const h4 *>(&sm.dUT[r][16 * kb + 4 * g]);
                    nd = mfma16x16x16_f16(aw, bu, nd);
                    const h4 aq = *reinterpret_cast<const h4 *>(QgT + co_idx<kChunk>(16 * ct + r, 16 * kb + 4 * g));
                    const h4 bo = *reinterpret_cast<const h4 *>(&sm.dOT[slot][r][16 * kb + 4 * g]);
                    nq = mfma16x16x16_f16(aq, bo, nq);
                }
                dS[t] = nd + a.scale * nq;
            }
            lds_barrier();
        }
    }
    if (a.dh0) {
        float *d0 = a.dh0 + (n * H + h) * (int64_t)(kK * kV) + col0 + r;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) d0[(16 * (2 * w + t) + 4 * g + e) * kV] = dS[t][e];
    }
}

// ---- 4. the per-chunk gradient -----------------------------------------------

constexpr int kMainQ = 4;                      // column groups
constexpr int kMainThreads = 256 * kMainQ;     // waves: row block w = wave & 3, column group cq = wave >> 2
constexpr int kMainNC = 8 / kMainQ;            // 16-column tiles of a wave in the 64 x 128 results
constexpr int kMainJT = 4 / kMainQ;            // 16-column tiles of a wave in the 64 x 64 results
constexpr int kMainSegs = kMainThreads / kK;   // row segments of the reverse cumulative sum
constexpr int kMainTPR = kMainThreads / kK;    // threads per state row when staging dS'
constexpr int kRP = 132;           // row pitch of the 128-column tiles
constexpr int kTP = 68;            // row pitch of the 64 x 64 tiles

struct MainSmem {
    float U[kChunk][kRP];   // gamma Khat (P1), Ut (P2-P6), khat (P7), then dG and its reverse cumulative sum
    float Z[kChunk][kRP];   // Diag(b) Y (P1-P2), dUt (P3), Z (P3-P6), G (P7)
    float SB[kK][kRP];      // S (P1-P4), dS' (P5); in P7 dM in rows 0..63 and qhat in rows 64..127
    union {
        float T[kChunk][kTP];        // T (P0-P3)
        uint16_t D[kChunk][136];     // dO, bf16 (P4-P6)
    } t;
    float b[kChunk];
    float rq[kChunk], rk[kChunk];  // reciprocal norms of the rows of q and k (0 past the end)
    float db[kMainQ][kChunk];      // per column group
    float rs[2][kMainQ][kChunk];   // row sums qhat . dqhat and khat . dkhat, per column group
    float red[4][kK];       // column sums per row block
    float gns[kK];          // exp(G_n) * sum_v S * dS'
    float tot[kMainSegs][kK];      // segment totals of the reverse cumulative sum
    float pa[4 * kMainQ];          // per-wave dA_log sums
};

// The same pointer, hidden from the compiler: loads through it are not merged
// with loads of the same addresses in other phases, which would keep those
// values alive (in registers) across the whole kernel.  It stays a global
// (address space 1) pointer, so that the loads take a scalar base and a 32-bit
// offset instead of a 64-bit flat address per element.
typedef const __attribute__((address_space(1))) float gfloat;
__device__ __forceinline__ gfloat *__restrict__ opaque(const float *p) {
    asm volatile("" : "+s"(p));
    return (gfloat *)p;
}

// Staging of [kRows][128] fp32 row-major blocks from global memory into LDS
// tiles of pitch kRP, 16 bytes per thread and pass: load() issues every load
// of the block into registers, store() writes them (after the caller's other
// loads, so that the latencies overlap rather than add up).
template <int kRows>
struct RowStage {
    static constexpr int kN = kRows * 32 / kMainThreads;
    float4 v[kN];
    __device__ __forceinline__ void load(const float *src, int tid) {
#pragma unroll
        for (int n = 0; n < kN; ++n) {
            const int idx = tid + n * kMainThreads;
            v[n] = *reinterpret_cast<const float4 *>(src + (idx >> 5) * 128 + (idx & 31) * 4);
        }
    }
    __device__ __forceinline__ void store(float (*dst)[kRP], int tid) const {
#pragma unroll
        for (int n = 0; n < kN; ++n) {
            const int idx = tid + n * kMainThreads;
            const int i = idx >> 5, c4 = (idx & 31) * 4;
            dst[i][c4] = v[n].x;
            dst[i][c4 + 1] = v[n].y;
            dst[i][c4 + 2] = v[n].z;
            dst[i][c4 + 3] = v[n].w;
        }
    }
};

// Staging of the 128 x 128 fp32 state the forward's chain saved in its register
// layout ([16-column block][16-row tile ct][lane][e]: lane (r, g) holds rows
// 16 ct + 4 g + e of column 16 block + r) into an LDS tile of pitch kRP,
// 16 bytes per thread and pass, loads first as in RowStage.
struct StateStage {
    static constexpr int kN = kK * kV / 4 / kMainThreads;
    float4 v[kN];
    __device__ __forceinline__ void load(const float *src, int tid) {
#pragma unroll
        for (int n = 0; n < kN; ++n) v[n] = reinterpret_cast<const float4 *>(src)[tid + n * kMainThreads];
    }
    __device__ __forceinline__ void store(float (*dst)[kRP], int tid) const {
#pragma unroll
        for (int n = 0; n < kN; ++n) {
            const int idx = tid + n * kMainThreads;
            const int ln = idx & 63;
            const int row = 16 * ((idx >> 6) & 7) + 4 * (ln >> 4), col = 16 * (idx >> 9) + (ln & 15);
            dst[row][col] = v[n].x;
            dst[row + 1][col] = v[n].y;
            dst[row + 2][col] = v[n].z;
            dst[row + 3][col] = v[n].w;
        }
    }
};
static_assert(StateStage::kN * kMainThreads * 4 == kK * kV, "StateStage covers the state exactly");

// Keep the accumulators' current values in registers here: without this the
// compiler sinks a phase's updates into the last phase that reads them, and
// the operands it keeps alive for that (loaded values, products) run out of
// registers and are spilled.
template <int kN>
__device__ __forceinline__ void pin(f4 (&x)[kN]) {
#pragma unroll
    for (int i = 0; i < kN; ++i) asm volatile("" : "+v"(x[i]));
}

// One thread's share of a [64][128] tile of normalised rows, x_i / |x_i| from the
// bf16 input rows and the reciprocal norms: row tid / 16, columns 8 (tid % 16) .. + 7.
// Rows past the end read row 0 (in bounds) and have a reciprocal norm of 0.
struct NormRow {
    uint4 raw;
    int row, c8;
    __device__ __forceinline__ void load(const uint16_t *x, int64_t t0, int64_t H, int64_t h, int L, int tid) {
        row = tid >> 4;
        c8 = 8 * (tid & 15);
        raw = *reinterpret_cast<const uint4 *>(x + ((t0 + (row < L ? row : 0)) * H + h) * kK + c8);
    }
    // the 8 values times rn, each times f[e] when given
    __device__ __forceinline__ void store(float (*dst)[kRP], float rn, const float *f = nullptr) const {
        float x[8];
        unpack_bf16x8(raw, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float v = x[e] * rn;
            dst[row][c8 + e] = f ? v * f[e] : v;
        }
    }
};

__global__ __launch_bounds__(kMainThreads, 1) void kda_bwd_main_kernel(BwdArgs a) {
    __shared__ MainSmem sm;
    const int64_t ws = a.unit_base + blockIdx.x;
    const int64_t slot = ws / a.H, h = ws - slot * a.H;
    int64_t t0;
    int L;
    if (!chunk_rows(a, slot, t0, L)) return;
    const int64_t H = a.H;
    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int w = wv & 3, cq = wv >> 2;
    const int lane = tid & 63, r = lane & 15, gq = lane >> 4;
    // Every buffer the kernel touches is distinct, and saying so lets the compiler
    // issue the epilogues' loads ahead of their stores instead of one after another.
    const float *__restrict__ S = a.hs + ws * (int64_t)(kK * kV);
    const float *__restrict__ dSp = a.dhs + ws * (int64_t)(kK * kV);
    const float *__restrict__ dUt = a.dUt + ws * (int64_t)(kChunk * kV);
    const float *__restrict__ G_all = a.G + ws * (kChunk * kK);
    const float *__restrict__ G = G_all;
    const float *__restrict__ Mk = a.Mk + ws * (kChunk * kChunk);
    const float *__restrict__ Tm = a.Tm + ws * (kChunk * kChunk);
    const float *__restrict__ rqv = a.rq + ws * kChunk;
    const float *__restrict__ rkv = a.rk + ws * kChunk;
    const float *__restrict__ bbv = a.bb + ws * kChunk;
    const uint16_t *__restrict__ vin = a.v;
    const uint16_t *__restrict__ gin = a.g;
    const float *__restrict__ dtb_h = a.dt_bias + h * kK;
    float *__restrict__ dqo = a.dq;
    float *__restrict__ dko = a.dk;
    float *__restrict__ dvo = a.dv;
    float *__restrict__ dgo = a.dg;
    float *__restrict__ dbo = a.dbeta;
    float *__restrict__ part = a.part + ws * (kK + 1);
    const float scale = a.scale;
    // v[i][c] of this lane's elements (rows row0 + e, columns 16 (kMainNC cq + c) + r),
    // 0 past the end (read in bounds, at row 0); loaded ahead of the products that use them
    auto load_v = [&](float (&vv)[kMainNC][4]) {
#pragma unroll
        for (int c = 0; c < kMainNC; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * w + 4 * gq + e, d = 16 * (kMainNC * cq + c) + r;
                vv[c][e] = bf16_bits_to_f32(vin[((t0 + (i < L ? i : 0)) * H + h) * kV + d]);
            }
#pragma unroll
        for (int c = 0; c < kMainNC; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (16 * w + 4 * gq + e >= L) vv[c][e] = 0.f;
    };
    const int64_t HK = H * kK;
    const int64_t obase = (t0 * H + h) * kK;
    auto out_at = [&](int i, int d) -> int64_t { return obase + i * HK + d; };

    // wave (w, cq) owns rows 16 w .. 16 w + 15 and column tiles ct = kMainNC cq + c
    // (c < kMainNC) of every 64 x 128 result; lane (r, gq) holds rows 16 w + 4 gq + e
    // of column 16 ct + r.  The gradients of qhat, khat and G accumulate in
    // registers, each element in its owning lane.
    const int row0 = 16 * w + 4 * gq;  // + e
    f4 dG[kMainNC], dqh[kMainNC], dkh[kMainNC];
#pragma unroll
    for (int c = 0; c < kMainNC; ++c) { dG[c] = f4{0, 0, 0, 0}; dqh[c] = dG[c]; dkh[c] = dG[c]; }

    // P0: T, b, gamma Khat and S into LDS (every load issued first)
    {
        static_assert(kChunk * kChunk == 4 * kMainThreads, "one float4 of T per thread");
        const float4 tv = *reinterpret_cast<const float4 *>(Tm + 4 * tid);
        float bv = 0.f, rqr = 0.f, rkr = 0.f;
        if (tid < kChunk) { bv = bbv[tid]; rqr = rqv[tid]; rkr = rkv[tid]; }
        NormRow kr;
        kr.load(a.k, t0, H, h, L, tid);
        const float rkn = rkv[kr.row];
        const float4 g0 = *reinterpret_cast<const float4 *>(G + kr.row * kK + kr.c8);
        const float4 g1 = *reinterpret_cast<const float4 *>(G + kr.row * kK + kr.c8 + 4);
        StateStage ss;
        ss.load(S, tid);
        *reinterpret_cast<float4 *>(&sm.t.T[tid >> 4][4 * (tid & 15)]) = tv;
        if (tid < kChunk) {
            sm.b[tid] = bv;
            sm.rq[tid] = rqr;
            sm.rk[tid] = rkr;
#pragma unroll
            for (int g2 = 0; g2 < kMainQ; ++g2) sm.db[g2][tid] = 0.f;
        }
        const float gam[8] = {__expf(g0.x), __expf(g0.y), __expf(g0.z), __expf(g0.w),
                              __expf(g1.x), __expf(g1.y), __expf(g1.z), __expf(g1.w)};
        kr.store(sm.U, rkn, gam);  // gamma khat
        ss.store(sm.SB, tid);
    }
    __syncthreads();

    // P1: Diag(b) Y, Y = V - (gamma Khat) S
    {
        float vv[kMainNC][4];
        load_v(vv);
        f4 acc[kMainNC];
#pragma unroll
        for (int c = 0; c < kMainNC; ++c) acc[c] = f4{0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int k0 = 32 * ks + 8 * gq;
            s8 ah, al;
            split8(&sm.U[16 * w + r][k0], ah, al);
#pragma unroll
            for (int c = 0; c < kMainNC; ++c) {
                const int col = 16 * (kMainNC * cq + c) + r;
                float x[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = sm.SB[k0 + e][col];
                s8 bh, bl;
                split8r(x, bh, bl);
                acc[c] = mfma16x16x32_bf16(ah, bh, acc[c]);
                acc[c] = mfma16x16x32_bf16(ah, bl, acc[c]);
                acc[c] = mfma16x16x32_bf16(al, bh, acc[c]);
            }
        }
#pragma unroll
        for (int c = 0; c < kMainNC; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ii = row0 + e, d = 16 * (kMainNC * cq + c) + r;
                sm.Z[ii][d] = sm.b[ii] * (vv[c][e] - acc[c][e]);
            }
    }
    __syncthreads();
    // P2: Ut = T (Diag(b) Y); T[i][j] = 0 for j > i
    {
        f4 acc[kMainNC];
#pragma unroll
        for (int c = 0; c < kMainNC; ++c) acc[c] = f4{0, 0, 0, 0};
        // k = j < 32 (w + 2) / 2 covers j <= 16 w + 15 (the rest of T's row is zero)
        for (int ks = 0; ks < (w + 2) / 2; ++ks) {
            const int k0 = 32 * ks + 8 * gq;
            s8 th, tl;
            split8(&sm.t.T[16 * w + r][k0], th, tl);
#pragma unroll
            for (int c = 0; c < kMainNC; ++c) {
                const int col = 16 * (kMainNC * cq + c) + r;
                float x[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = sm.Z[k0 + e][col];
                s8 bh, bl;
                split8r(x, bh, bl);
                acc[c] = mfma16x16x32_bf16(th, bh, acc[c]);
                acc[c] = mfma16x16x32_bf16(th, bl, acc[c]);
                acc[c] = mfma16x16x32_bf16(tl, bh, acc[c]);
            }
        }
#pragma unroll
        for (int c = 0; c < kMainNC; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.U[row0 + e][16 * (kMainNC * cq + c) + r] = acc[c][e];
    }
    __syncthreads();
    {
        RowStage<kChunk> us;
        us.load(dUt, tid);
        us.store(sm.Z, tid);
    }
    __syncthreads();
    // P3: Z = T^T dUt; dv = Diag(b) Z; db += Z . v
    {
        float vv[kMainNC][4];
        load_v(vv);
        f4 acc[kMainNC];
#pragma unroll
        for (int c = 0; c < kMainNC; ++c) acc[c] = f4{0, 0, 0, 0};
        // k = i >= 32 (w / 2) covers i >= 16 w (T[i][j] is zero for i < j)
        for (int ks = w / 2; ks < 2; ++ks) {
            const int k0 = 32 * ks + 8 * gq;
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = sm.t.T[k0 + e][16 * w + r];
            s8 th, tl;
            split8r(y, th, tl);
#pragma unroll
            for (int c = 0; c < kMainNC; ++c) {
                const int col = 16 * (kMainNC * cq + c) + r;
                float x[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = sm.Z[k0 + e][col];
                s8 bh, bl;
                split8r(x, bh, bl);
                acc[c] = mfma16x16x32_bf16(th, bh, acc[c]);
                acc[c] = mfma16x16x32_bf16(th, bl, acc[c]);
                acc[c] = mfma16x16x32_bf16(tl, bh, acc[c]);
            }
        }
        __syncthreads();  // every wave has read dUt
        float dbp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < kMainNC; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ii = row0 + e, d = 16 * (kMainNC * cq + c) + r;
                const float z = acc[c][e];
                sm.Z[ii][d] = z;
                if (ii < L) {
                    dvo[((t0 + ii) * H + h) * kV + d] = sm.b[ii] * z;
                    dbp[e] += z * vv[c][e];
                }
            }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float s = sum16(dbp[e]);
            if (r == 0) sm.db[cq][row0 + e] += s;
        }
    }
    __syncthreads();
    // dO into the T area (rows past the end zero); 16 bytes per thread and pass
    for (int idx = tid; idx < kChunk * 16; idx += kMainThreads) {
        const int i = idx >> 4, c8 = (idx & 15) * 8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (i < L) v = *reinterpret_cast<const uint4 *>(a.dout + ((t0 + i) * H + h) * kV + c8);
        *reinterpret_cast<uint4 *>(&sm.t.D[i][c8]) = v;
    }
    __syncthreads();
    // P4: dQg = scale dO S^T and Zw = -Z S^T
    {
        gfloat *__restrict__ G = opaque(G_all);
        f4 aq[kMainNC], az[kMainNC];
#pragma unroll
        for (int c = 0; c < kMainNC; ++c) { aq[c] = f4{0, 0, 0, 0}; az[c] = aq[c]; }
        // bf16 16x16x32 products, lane (r, gq) holding k = 32 ks + 8 gq .. + 7: dO is bf16
        // already, S and Z are split into bf16 hi + lo (S twice, Z S^T three times: products
        // good to about 2^-16, the lo * lo term dropped)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int k0 = 32 * ks + 8 * gq;
            const s8 a1 = __builtin_bit_cast(s8, *reinterpret_cast<const uint4 *>(&sm.t.D[16 * w + r][k0]));
            s8 zh, zl;
            split8(&sm.Z[16 * w + r][k0], zh, zl);
#pragma unroll
            for (int c = 0; c < kMainNC; ++c) {
                s8 sh, sl;
                split8(&sm.SB[16 * (kMainNC * cq + c) + r][k0], sh, sl);
                aq[c] = mfma16x16x32_bf16(a1, sh, aq[c]);
                aq[c] = mfma16x16x32_bf16(a1, sl, aq[c]);
                az[c] = mfma16x16x32_bf16(zh, sh, az[c]);
                az[c] = mfma16x16x32_bf16(zh, sl, az[c]);
                az[c] = mfma16x16x32_bf16(zl, sh, az[c]);
            }
        }
        float dbp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < kMainNC; ++c) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ii = row0 + e, d = 16 * (kMainNC * cq + c) + r;
                const int64_t xi = ((t0 + (ii < L ? ii : 0)) * H + h) * kK + d;  // row 0 past the end
                const float qh = bf16_bits_to_f32(a.q[xi]) * sm.rq[ii], kh = bf16_bits_to_f32(a.k[xi]) * sm.rk[ii];
                const float gam = __expf(G[ii * kK + d]);
                const float bi = sm.b[ii];
                const float dQg = scale * aq[c][e], Zw = -az[c][e];
                dqh[c][e] = gam * dQg;
                dkh[c][e] = bi * gam * Zw;
                dG[c][e] += gam * qh * dQg + bi * gam * kh * Zw;
                dbp[e] += Zw * gam * kh;
            }
            // per column tile: its 12 loads are issued together, the next tile's after
            pin(dqh);
            pin(dkh);
            pin(dG);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float s = sum16(dbp[e]);
            if (r == 0) sm.db[cq][row0 + e] += s;
        }
    }
    __syncthreads();
    // dS' into LDS, over S; exp(G_n) sum_v S[d][v] dS'[d][v] on the way (kMainTPR threads per
    // state row, each reading S from LDS where it then writes dS')
    {
        constexpr int kCols = kV / kMainTPR;
        const int d = tid / kMainTPR, qt = tid % kMainTPR;
        const float *dr = dSp + d * kV + kCols * qt;
        float s = 0.f;
#pragma unroll
        for (int c4 = 0; c4 < kCols; c4 += 4) {
            const float4 x = *reinterpret_cast<const float4 *>(&sm.SB[d][kCols * qt + c4]);
            const float4 y = *reinterpret_cast<const float4 *>(dr + c4);
            s += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
            sm.SB[d][kCols * qt + c4] = y.x;
            sm.SB[d][kCols * qt + c4 + 1] = y.y;
            sm.SB[d][kCols * qt + c4 + 2] = y.z;
            sm.SB[d][kCols * qt + c4 + 3] = y.w;
        }
#pragma unroll
        for (int o = 1; o < kMainTPR; o <<= 1) s += __shfl_xor(s, o);
        if (qt == 0) sm.gns[d] = __expf(G[(L - 1) * kK + d]) * s;
    }
    __syncthreads();
    // P5: dKbar = Ut dS'^T
    {
        gfloat *__restrict__ G = opaque(G_all);
        f4 acc[kMainNC];
#pragma unroll
        for (int c = 0; c < kMainNC; ++c) acc[c] = f4{0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int k0 = 32 * ks + 8 * gq;
            s8 uh, ul;
            split8(&sm.U[16 * w + r][k0], uh, ul);
#pragma unroll
            for (int c = 0; c < kMainNC; ++c) {
                s8 dh, dl;
                split8(&sm.SB[16 * (kMainNC * cq + c) + r][k0], dh, dl);
                acc[c] = mfma16x16x32_bf16(uh, dh, acc[c]);
                acc[c] = mfma16x16x32_bf16(uh, dl, acc[c]);
                acc[c] = mfma16x16x32_bf16(ul, dh, acc[c]);
            }
        }
#pragma unroll
        for (int c = 0; c < kMainNC; ++c) {
            const int d = 16 * (kMainNC * cq + c) + r;
            const float Gn = G[(L - 1) * kK + d];
            float colp = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ii = row0 + e;
                const float eK = __expf(Gn - G[ii * kK + d]);
                const int64_t xi = ((t0 + (ii < L ? ii : 0)) * H + h) * kK + d;  // row 0 past the end
                const float kb = eK * (bf16_bits_to_f32(a.k[xi]) * sm.rk[ii]);
                const float dkb = acc[c][e];
                dkh[c][e] += eK * dkb;
                dG[c][e] -= kb * dkb;
                colp += kb * dkb;
            }
            colp = sum4g(colp);
            if (gq == 0) sm.red[w][d] = colp;
        }
        pin(dkh);
        pin(dG);
    }
    __syncthreads();
    // P6: dA_qk = scale dO Ut^T (j <= i), dA_kk = -Z Ut^T (j < i); db += dA_kk . M;
    // dM = Diag(b) dA_kk.  Wave (w, cq) takes column tiles jt = kMainJT cq + jj.
    {
        f4 accA[kMainJT], accK[kMainJT];
#pragma unroll
        for (int jj = 0; jj < kMainJT; ++jj) { accA[jj] = f4{0, 0, 0, 0}; accK[jj] = accA[jj]; }
        if (kMainJT * cq <= w) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int k0 = 32 * ks + 8 * gq;
                const s8 a1 = __builtin_bit_cast(s8, *reinterpret_cast<const uint4 *>(&sm.t.D[16 * w + r][k0]));
                s8 zh, zl;
                split8(&sm.Z[16 * w + r][k0], zh, zl);
#pragma unroll
                for (int jj = 0; jj < kMainJT; ++jj) {
                    const int jt = kMainJT * cq + jj;
                    if (jt <= w) {
                        s8 uh, ul;
                        split8(&sm.U[16 * jt + r][k0], uh, ul);
                        accA[jj] = mfma16x16x32_bf16(a1, uh, accA[jj]);
                        accA[jj] = mfma16x16x32_bf16(a1, ul, accA[jj]);
                        accK[jj] = mfma16x16x32_bf16(zh, uh, accK[jj]);
                        accK[jj] = mfma16x16x32_bf16(zh, ul, accK[jj]);
                        accK[jj] = mfma16x16x32_bf16(zl, uh, accK[jj]);
                    }
                }
            }
        }
        float dbp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jj = 0; jj < kMainJT; ++jj)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int jt = kMainJT * cq + jj;
                const int ii = row0 + e, j = 16 * jt + r;
                const float dAq = (jt <= w && j <= ii) ? scale * accA[jj][e] : 0.f;
                const float dAk = (jt <= w && j < ii) ? -accK[jj][e] : 0.f;
                dbp[e] += dAk * Mk[ii * kChunk + j];
                sm.SB[ii][64 + j] = dAq;
                sm.SB[ii][j] = sm.b[ii] * dAk;
            }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float s = sum16(dbp[e]);
            if (r == 0) sm.db[cq][row0 + e] += s;
        }
    }
    __syncthreads();
    // khat, G and qhat into LDS for the Gram gradients
    {
        NormRow kr, qr;
        kr.load(a.k, t0, H, h, L, tid);
        qr.load(a.q, t0, H, h, L, tid);
        RowStage<kChunk> gs;
        gs.load(G, tid);
        kr.store(sm.U, sm.rk[kr.row]);
        qr.store(&sm.SB[kChunk], sm.rq[qr.row]);
        gs.store(sm.Z, tid);
    }
    __syncthreads();
    // P7: the decayed Gram matrices P[i][j] = sum_d x_i y_j exp(G_i - G_j): for M
    // (x = y = khat, gradient dM) and A_qk (x = qhat, y = khat, gradient dA_qk).  These stay on
    // the fp32 matrix cores: the gate's gradient is a difference of these decay-weighted sums,
    // which cancel, and bf16 hi + lo products (about 2^-16) put dA_log past 5e-3 relative.
    {
        const float(*kh)[kRP] = sm.U;
        const float(*Gs)[kRP] = sm.Z;
        const float(*qh)[kRP] = &sm.SB[kChunk];
        float refc[kMainNC];  // G at the reference row 16 w + 8, this lane's columns
#pragma unroll
        for (int c = 0; c < kMainNC; ++c) refc[c] = Gs[16 * w + 8][16 * (kMainNC * cq + c) + r];
        // rows i of block w: sum_{j <= 16 w + 15} dP[i][j] y_j exp(ref - G_j), times exp(G_i - ref)
        {
            f4 rm[kMainNC], ra[kMainNC];
#pragma unroll
            for (int c = 0; c < kMainNC; ++c) { rm[c] = f4{0, 0, 0, 0}; ra[c] = rm[c]; }
#pragma unroll 2
            for (int ks = 0; ks < 4 * (w + 1); ++ks) {
                const int j = 4 * ks + gq;
                const float a1 = sm.SB[16 * w + r][j], a2 = sm.SB[16 * w + r][64 + j];
#pragma unroll
                for (int c = 0; c < kMainNC; ++c) {
                    const int d = 16 * (kMainNC * cq + c) + r;
                    const float bv = kh[j][d] * __expf(refc[c] - Gs[j][d]);
                    rm[c] = mma(a1, bv, rm[c]);
                    ra[c] = mma(a2, bv, ra[c]);
                }
            }
#pragma unroll
            for (int c = 0; c < kMainNC; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int ii = row0 + e, d = 16 * (kMainNC * cq + c) + r;
                    const float s = __expf(Gs[ii][d] - refc[c]);
                    const float RxM = rm[c][e] * s, RxA = ra[c][e] * s;
                    dkh[c][e] += RxM;
                    dqh[c][e] += RxA;
                    dG[c][e] += kh[ii][d] * RxM + qh[ii][d] * RxA;
                }
        }
        // columns j of block w: sum_{i >= 16 w} (dM[i][j] khat_i + dA_qk[i][j] qhat_i) exp(G_i - ref),
        // times exp(ref - G_j)
        {
            f4 ry[kMainNC];
#pragma unroll
            for (int c = 0; c < kMainNC; ++c) ry[c] = f4{0, 0, 0, 0};
#pragma unroll 2
            for (int ks = 4 * w; ks < 16; ++ks) {
                const int i = 4 * ks + gq;
                const float a1 = sm.SB[i][16 * w + r], a2 = sm.SB[i][64 + 16 * w + r];
#pragma unroll
                for (int c = 0; c < kMainNC; ++c) {
                    const int d = 16 * (kMainNC * cq + c) + r;
                    const float eg = __expf(Gs[i][d] - refc[c]);
                    ry[c] = mma(a1, kh[i][d] * eg, ry[c]);
                    ry[c] = mma(a2, qh[i][d] * eg, ry[c]);
                }
            }
#pragma unroll
            for (int c = 0; c < kMainNC; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int jj = row0 + e, d = 16 * (kMainNC * cq + c) + r;
                    const float Ry = ry[c][e] * __expf(refc[c] - Gs[jj][d]);
                    dkh[c][e] += Ry;
                    dG[c][e] -= kh[jj][d] * Ry;
                }
        }
    }
    __syncthreads();
    // P8: dG_n into the last valid row, then da_t = sum_{i >= t} dG_i
#pragma unroll
    for (int c = 0; c < kMainNC; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int ii = row0 + e, d = 16 * (kMainNC * cq + c) + r;
            float v = dG[c][e];
            if (ii == L - 1) v += sm.gns[d] + sm.red[0][d] + sm.red[1][d] + sm.red[2][d] + sm.red[3][d];
            sm.Z[ii][d] = ii < L ? v : 0.f;
        }
    __syncthreads();
    {  // kMainSegs threads per column, each a segment of rows: sums within the segment, then the
       // later segments' totals
        constexpr int kSR = kChunk / kMainSegs;
        const int d = tid & (kK - 1), sg = tid / kK;
        float run = 0.f;
#pragma unroll
        for (int i = kSR * sg + kSR - 1; i >= kSR * sg; --i) {
            run += sm.Z[i][d];
            sm.Z[i][d] = run;
        }
        sm.tot[sg][d] = run;
        __syncthreads();
        float carry = 0.f;
        for (int s2 = sg + 1; s2 < kMainSegs; ++s2) carry += sm.tot[s2][d];
#pragma unroll
        for (int i = kSR * sg; i < kSR * sg + kSR; ++i) sm.Z[i][d] += carry;
    }
    // P9: norms, gate, outputs.  Row sums of qhat . dqhat and khat . dkhat first
    // (khat and qhat are still in LDS from P7).
    {
    const float(*kh)[kRP] = sm.U;
    const float(*qh)[kRP] = &sm.SB[kChunk];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int ii = row0 + e;
        float a1 = 0.f, a2 = 0.f;
        if (ii < L) {
#pragma unroll
            for (int c = 0; c < kMainNC; ++c) {
                const int d = 16 * (kMainNC * cq + c) + r;
                a1 += qh[ii][d] * dqh[c][e];
                a2 += kh[ii][d] * dkh[c][e];
            }
        }
        a1 = sum16(a1);
        a2 = sum16(a2);
        if (r == 0) {
            sm.rs[0][cq][ii] = a1;
            sm.rs[1][cq][ii] = a2;
        }
    }
    __syncthreads();
    {
        const float nA = -expf(a.A_log[h]);
        // branch-free, so that the loads (rows past the end read at row 0, their results
        // unused) are issued together rather than each inside its row's condition
        float rqe[4], rke[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int il = row0 + e < L ? row0 + e : 0;
            rqe[e] = sm.rq[il];
            rke[e] = sm.rk[il];
        }
        float pa = 0.f;
#pragma unroll
        for (int c = 0; c < kMainNC; ++c) {
            const int d = 16 * (kMainNC * cq + c) + r;
            const float dtb = dtb_h[d];
            float xg[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int il = row0 + e < L ? row0 + e : 0;
                xg[e] = bf16_bits_to_f32(gin[out_at(il, d)]) + dtb;
            }
            float colp = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ii = row0 + e;
                const bool valid = ii < L;
                float sq = 0.f, sk = 0.f;
#pragma unroll
                for (int g2 = 0; g2 < kMainQ; ++g2) { sq += sm.rs[0][g2][ii]; sk += sm.rs[1][g2][ii]; }
                const float dq = rqe[e] * (dqh[c][e] - sq * qh[ii][d]);
                const float dk = rke[e] * (dkh[c][e] - sk * kh[ii][d]);
                const float z = nA * softplus_fast(xg[e]);
                const float da = sm.Z[ii][d];
                const bool open = valid && z > a.lower_bound;  // the gate is not clamped
                const float dx = open ? da * nA * sigmoid_fast(xg[e]) : 0.f;
                pa += open ? da * z : 0.f;
                colp += dx;
                if (valid) {
                    const int64_t o = out_at(ii, d);
                    dqo[o] = dq;
                    dko[o] = dk;
                    dgo[o] = dx;
                }
            }
            colp = sum4g(colp);
            if (gq == 0) sm.red[w][d] = colp;
        }
        pa = sum4g(sum16(pa));
        if (lane == 0) sm.pa[wv] = pa;
    }
    }
    __syncthreads();
    if (tid < kK) part[tid] = sm.red[0][tid] + sm.red[1][tid] + sm.red[2][tid] + sm.red[3][tid];
    if (tid == kK) {
        float s = 0.f;
        for (int i = 0; i < 4 * kMainQ; ++i) s += sm.pa[i];
        part[kK] = s;
    }
    if (tid < L) {
        const float b = sm.b[tid];
        float dbs = 0.f;
#pragma unroll
        for (int g2 = 0; g2 < kMainQ; ++g2) dbs += sm.db[g2][tid];
        dbo[(t0 + tid) * H + h] = dbs * b * (1.f - b);
    }
}

// ---- 5. the shared parameters ------------------------------------------------

// One 1024-thread workgroup per head: thread (slice j, column c) sums column c
// (c < K: dt_bias channel c; c = K: A_log) over the chunk slots j, j + 7, j + 14,
// ... in increasing order, eight loads in flight, then the seven slice sums are
// added in slice order: a fixed order, so the result is the same bits on every
// call.  (One thread per column would wait out one load per chunk in turn.)
constexpr int kParamThreads = 1024;
constexpr int kParamSlices = kParamThreads / (kK + 1);  // 7

__global__ __launch_bounds__(kParamThreads) void kda_bwd_params_kernel(BwdArgs a) {
    __shared__ double red[kParamSlices][kK + 1];
    const int64_t h = blockIdx.x;
    const int tid = threadIdx.x;
    const int j = tid / (kK + 1), c = tid - j * (kK + 1);
    const int64_t total = a.cu ? (int64_t)a.chunk_off[a.N] : a.slots;
    if (j < kParamSlices) {
        const float *p = a.part + h * (kK + 1) + c;
        const int64_t step = a.H * (kK + 1);  // one slot
        double s = 0.0;
        int64_t slot = j;
        for (; slot + 7 * kParamSlices < total; slot += 8 * kParamSlices) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = p[(slot + u * kParamSlices) * step];
#pragma unroll
            for (int u = 0; u < 8; ++u) s += (double)v[u];
        }
        for (; slot < total; slot += kParamSlices) s += (double)p[slot * step];
        red[j][c] = s;
    }
    __syncthreads();
    if (tid <= kK) {
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < kParamSlices; ++i) s += red[i][tid];
        if (tid < kK) a.ddt_bias[h * kK + tid] = (float)s;
        else a.dA_log[h] = (float)s;
    }
}

}  // namespace

hipError_t kda_launch_bwd_prep(const BwdArgs &a0, hipStream_t s) {
    BwdArgs a = a0;
    const int64_t units = a.slots * a.H;
    const int64_t piece = launch_piece(kMaxUnitsPerLaunch, a.piece_cap);
    for (int64_t u0 = 0; u0 < units; u0 += piece) {
        a.unit_base = u0;
        const int64_t nu = units - u0 < piece ? units - u0 : piece;
        hipLaunchKernelGGL(kda_bwd_prep_kernel, dim3((unsigned)nu), dim3(kThreads), 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t kda_launch_bwd_chain(const BwdArgs &a0, hipStream_t s) {
    BwdArgs a = a0;
    const int64_t NH = a.N * a.H;
    const int64_t groups = (NH + 7) / 8;
    const int64_t gpiece = launch_piece(kMaxGroupsPerLaunch, a.piece_cap);
    for (int64_t g0 = 0; g0 < groups; g0 += gpiece) {
        a.chain_base = 8 * g0;
        const int64_t ng = groups - g0 < gpiece ? groups - g0 : gpiece;
        hipLaunchKernelGGL(kda_bwd_chain_kernel, dim3((unsigned)(ng * 64)), dim3(64 * kChainWaves), 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t kda_launch_bwd_grad(const BwdArgs &a0, hipStream_t s) {
    BwdArgs a = a0;
    const int64_t units = a.slots * a.H;
    const int64_t piece = launch_piece(kMaxUnitsPerLaunch, a.piece_cap);
    for (int64_t u0 = 0; u0 < units; u0 += piece) {
        a.unit_base = u0;
        const int64_t nu = units - u0 < piece ? units - u0 : piece;
        hipLaunchKernelGGL(kda_bwd_main_kernel, dim3((unsigned)nu), dim3(kMainThreads), 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kda_bwd_params_kernel, dim3((unsigned)a.H), dim3(kParamThreads), 0, s, a);
    return hipGetLastError();
}
