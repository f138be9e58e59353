// kda_intra_body.h -- the per-(chunk, head) work of the intra-chunk kernel,
// shared by the stand-alone intra kernel (kda_intra.hip) and the producer
// workgroups of the pipelined forward (kda_fused.hip).  Internal header.
//
// intra_chunk() is the whole computation for one 64-token chunk of one head
// on 256 threads (four waves); the caller supplies the chunk slot, the head,
// the LDS area and the barrier that orders LDS traffic between those four
// waves (the workgroup barrier in the stand-alone kernel, a barrier over one
// half of the workgroup in the pipelined one).  See kda_intra.hip for the
// method.
#pragma once
#include "kda_common.h"

namespace kda {
namespace intra {

constexpr int kThreads = 256;
constexpr int kYP = 132;   // row pitch (floats) of the decayed-key rows
constexpr int kLP = 68;    // row pitch (floats) of A_kk / T
constexpr int kTP = 72;    // row pitch (halves) of the transposed operands and of T in fp16
constexpr float kLog2e = 1.4426950408889634f;

struct __align__(16) IntraSmem {
    union {
        float yt[64 * kYP];  // Y_j = exp(G_{r-1} - G_j) * khat_j, r = start of j's 16-row block
        struct {
            _Float16 kg[128 * kTP];  // (b * gamma * khat)^T   [channel][token]
            _Float16 vb[128 * kTP];  // (b * v)^T              [value column][token]
        } t;
    } u;
    float L[64 * kLP];      // b-scaled A_kk (strictly lower); diagonal blocks overwritten by T
    _Float16 Th[64 * kTP];  // T = (I + A_kk)^-1 in fp16, zeros above the diagonal
    float pblk[4 * 128];    // per 16-row block: product of the block's decays, per channel
};

__device__ __forceinline__ h4 to_h4(const f4 &x) {
    h4 r;
    r[0] = (_Float16)x[0]; r[1] = (_Float16)x[1]; r[2] = (_Float16)x[2]; r[3] = (_Float16)x[3];
    return r;
}

__device__ __forceinline__ h8 to_h8(const f4 &a, const f4 &b) {
    h8 r;
    r[0] = (_Float16)a[0]; r[1] = (_Float16)a[1]; r[2] = (_Float16)a[2]; r[3] = (_Float16)a[3];
    r[4] = (_Float16)b[0]; r[5] = (_Float16)b[1]; r[6] = (_Float16)b[2]; r[7] = (_Float16)b[3];
    return r;
}

// A 16-byte intermediate store, with the non-temporal hint when kStream: the
// state chain reads the line once, from HBM, much later.
template <bool kStream>
__device__ __forceinline__ void store_h8(_Float16 *p, const h8 &v) {
    if constexpr (kStream) __builtin_nontemporal_store(v, reinterpret_cast<h8 *>(p));
    else *reinterpret_cast<h8 *>(p) = v;
}

// fp16 hi + lo split of four floats.
__device__ __forceinline__ void split_h4(const f4 &x, h4 &hi, h4 &lo) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const _Float16 h = (_Float16)x[e];
        hi[e] = h;
        lo[e] = (_Float16)(x[e] - (float)h);
    }
}

// a * b with both operands split into fp16 hi + lo (three MFMAs, ~22-bit products).
__device__ __forceinline__ f4 mfma_split16(const f4 &a, const f4 &b, f4 c) {
    h4 ah, al, bh, bl;
    split_h4(a, ah, al);
    split_h4(b, bh, bl);
    c = mfma16x16x16_f16(ah, bh, c);
    c = mfma16x16x16_f16(ah, bl, c);
    c = mfma16x16x16_f16(al, bh, c);
    return c;
}

// Off-diagonal blocks of T = (I + A_kk)^-1 in column block J (wave J):
//   T_ij = -T_ii * sum_{k=j}^{i-1} L_ik T_kj   (16x16 blocks, split-fp16 MFMA),
// with the column's blocks kept in registers in accumulator layout
// (Tc[k][e] = T[16 k + 4 cg + e][16 J + r16]), which is also their B-operand layout.
template <int J>
__device__ __forceinline__ void offdiag_column(IntraSmem &sm, int r16, int cg) {
    f4 Tc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) Tc[J][e] = sm.L[(16 * J + 4 * cg + e) * kLP + 16 * J + r16];
#pragma unroll
    for (int ib = J + 1; ib < 4; ++ib) {
        f4 R = f4{0, 0, 0, 0};
#pragma unroll
        for (int kb = J; kb < ib; ++kb) {
            const f4 la = *reinterpret_cast<const f4 *>(&sm.L[(16 * ib + r16) * kLP + 16 * kb + 4 * cg]);
            R = mfma_split16(la, Tc[kb], R);
        }
        const f4 ta = *reinterpret_cast<const f4 *>(&sm.L[(16 * ib + r16) * kLP + 16 * ib + 4 * cg]);
        Tc[ib] = -mfma_split16(ta, R, f4{0, 0, 0, 0});
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.Th[(16 * ib + 4 * cg + e) * kTP + 16 * J + r16] = (_Float16)Tc[ib][e];
    }
}


// A 16-byte input load; with kNT the non-temporal hint (the line is read once
// and should not displace other data from L2).
template <bool kNT>
__device__ __forceinline__ uint4 load_in(const uint16_t *p) {
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    if constexpr (kNT) {
        const u4 v = __builtin_nontemporal_load(reinterpret_cast<const u4 *>(p));
        return make_uint4(v[0], v[1], v[2], v[3]);
    } else {
        return *reinterpret_cast<const uint4 *>(p);
    }
}

// One chunk of one head: computes and stores -W, Q_gamma, Kbar^T, A_qk, U
// (fp16 fragments) and exp(G_n) for chunk slot `slot` and head `h`.  `tid` is
// the thread's index among the 256 threads that share `sm`; bar() must order
// LDS accesses among exactly those threads.  For a packed batch a slot past
// the last chunk returns at once (no barrier is reached).
template <bool kStream, typename Bar, bool kStreamIn = false>
__device__ __forceinline__ void intra_chunk(const IntraArgs &a, int64_t slot, int64_t h, IntraSmem &sm, int tid,
                                            Bar &&bar) {
    const int64_t H = a.H;

    // ---- which tokens this chunk covers -----------------------------------
    int64_t t0;  // first token row on the flattened [B*T] axis
    int L;       // valid rows (1..64)
    if (a.cu) {
        const int64_t total = a.chunk_off[a.N];
        if (slot >= total) return;
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

    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave = 16-row block (wave-uniform)
    const int lane = tid & 63;
    const int r16 = lane & 15;       // row within the block
    const int cg = lane >> 4;        // 8-channel group within each 32-channel step
    const int row = 16 * w + r16;
    const bool valid = row < L;

    const int64_t ws = slot * H + h;  // workspace index of this (chunk, head)

    // ---- P0: load, normalise, gate, block-local decay products ------------
    // Loads are issued dt_bias and g first (rows past the end reload the last
    // row, zeroed below): they complete in order, so the gate math starts as
    // soon as these arrive while q, k, v are still in flight.
    uint4 graw[4], kraw[4], qraw[4], vraw[4];
    float4 dtb4[8];  // dt_bias[h][32 kk + 8 cg + 0..7] as two float4 per kk
    float bl;
    {
        const int64_t base = ((t0 + (valid ? row : L - 1)) * H + h) * kK;
        const float *dtb = a.dt_bias + h * kK;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            dtb4[2 * kk] = *reinterpret_cast<const float4 *>(dtb + 32 * kk + 8 * cg);
            dtb4[2 * kk + 1] = *reinterpret_cast<const float4 *>(dtb + 32 * kk + 8 * cg + 4);
        }
        bl = bf16_bits_to_f32(a.beta[(t0 + (valid ? row : L - 1)) * H + h]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) graw[kk] = load_in<kStreamIn>(a.g + base + 32 * kk + 8 * cg);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) kraw[kk] = load_in<kStreamIn>(a.k + base + 32 * kk + 8 * cg);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qraw[kk] = load_in<kStreamIn>(a.q + base + 32 * kk + 8 * cg);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) vraw[kk] = load_in<kStreamIn>(a.v + base + 32 * kk + 8 * cg);
        // every load is issued before any of them is used: otherwise the
        // scheduler starts unpacking g early, and the register reuse that
        // follows makes the k, q, v loads wait for the first g load to land
        __builtin_amdgcn_sched_barrier(0);
    }

    // gate in base 2: log2 d = log2e max(lb, -exp(A_log) softplus(x)), x = g + dt_bias
    // (gate_log2), i.e. d = exp(max(lb, -exp(A_log) softplus(x))); then the inclusive product
    // over the block's rows: P_i = exp(G_i - G_{r-1}).
    float P[32];
    {
        const float nA = -fast_exp(a.A_log[h]);
        const float lb2 = a.lower_bound * kLog2e;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const float4 d0 = dtb4[2 * kk], d1 = dtb4[2 * kk + 1];
            const float db[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
            float gf[8];
            unpack_bf16x8(graw[kk], gf);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float l2 = gate_log2(gf[e] + db[e], nA, lb2);
                P[8 * kk + e] = valid ? l2 : 0.0f;  // log2 of the decay
            }
        }
    }
    // inclusive prefix sums of the log2 decays over the block's rows (one DPP
    // row = 16 lanes = the block), then P = 2^sum; one DPP add per step
#pragma unroll
    for (int s = 1; s < 16; s <<= 1) {
#pragma unroll
        for (int e = 0; e < 32; ++e) P[e] += dpp_row_shr_zero(P[e], s);
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) P[e] = __builtin_amdgcn_exp2f(P[e]);
    // L2 norms (rows past the end are zeroed: no key, no query, b = 0)
    if (!valid) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            kraw[kk] = make_uint4(0, 0, 0, 0); qraw[kk] = kraw[kk]; vraw[kk] = kraw[kk];
        }
    }
    float qv[32], kv[32];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        unpack_bf16x8(kraw[kk], kv + 8 * kk);
        unpack_bf16x8(qraw[kk], qv + 8 * kk);
    }
    float ssq = 0.f, ssk = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) { ssq += qv[e] * qv[e]; ssk += kv[e] * kv[e]; }
    ssq += __shfl_xor(ssq, 16); ssq += __shfl_xor(ssq, 32);
    ssk += __shfl_xor(ssk, 16); ssk += __shfl_xor(ssk, 32);
    const float rq = fast_rsqrt(ssq + 1e-6f);
    const float rk = fast_rsqrt(ssk + 1e-6f);
    const float b = valid ? fast_rcp(1.0f + fast_exp(-bl)) : 0.f;

    // X_i = P_i khat_i and Q'_i = P_i qhat_i stay in registers; Y_j = khat_j / P_j
    // (<= exp(80) khat_j) goes to LDS; P becomes the block total pe.
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        float yv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int idx = 8 * kk + e;
            const float pe = dpp_row_bcast15(P[idx]);
            const float kh = kv[idx] * rk;
            yv[e] = kh * fast_rcp(P[idx]);
            kv[idx] = kh * P[idx];          // X
            qv[idx] = qv[idx] * rq * P[idx];  // Q'
            P[idx] = pe;
        }
        float4 *dst = reinterpret_cast<float4 *>(&sm.u.yt[row * kYP + 32 * kk + 8 * cg]);
        dst[0] = make_float4(yv[0], yv[1], yv[2], yv[3]);
        dst[1] = make_float4(yv[4], yv[5], yv[6], yv[7]);
    }
    // b v in fp16 (natural layout)
    h8 vbF[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        float vf[8];
        unpack_bf16x8(vraw[kk], vf);
#pragma unroll
        for (int e = 0; e < 8; ++e) vbF[kk][e] = (_Float16)(b * vf[e]);
    }
    if (r16 == 0) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            float4 *dst = reinterpret_cast<float4 *>(&sm.pblk[w * 128 + 32 * kk + 8 * cg]);
            dst[0] = make_float4(P[8 * kk + 0], P[8 * kk + 1], P[8 * kk + 2], P[8 * kk + 3]);
            dst[1] = make_float4(P[8 * kk + 4], P[8 * kk + 5], P[8 * kk + 6], P[8 * kk + 7]);
        }
    }
    bar();  // B1: block totals and decayed key rows visible

    // ---- P1: cross-block decays, chunk outputs, Gram tiles ----------------
    // The 0/1 selection matrices: lane (r, g) slot j is 1 where 8 g + j == r + 16 half.
    h8 sel[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int j = 0; j < 8; ++j) sel[hf][j] = (8 * cg + j == r16 + 16 * hf) ? (_Float16)1.0f : (_Float16)0.0f;

    h8 kgF[4];                          // b gamma khat (natural layout, fp16)
    f4 akk_o[3], aqk_o[3], akk_d = f4{0, 0, 0, 0}, aqk_d = f4{0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < 3; ++t) { akk_o[t] = f4{0, 0, 0, 0}; aqk_o[t] = f4{0, 0, 0, 0}; }
    _Float16 *Kf = a.Kf + ws * kKfElems;
    _Float16 *Qf = a.Qf + ws * kQfElems;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int c0 = 32 * kk + 8 * cg;
        float pb[4][8];
#pragma unroll
        for (int wp = 0; wp < 4; ++wp) {
            const float4 x0 = *reinterpret_cast<const float4 *>(&sm.pblk[wp * 128 + c0]);
            const float4 x1 = *reinterpret_cast<const float4 *>(&sm.pblk[wp * 128 + c0 + 4]);
            pb[wp][0] = x0.x; pb[wp][1] = x0.y; pb[wp][2] = x0.z; pb[wp][3] = x0.w;
            pb[wp][4] = x1.x; pb[wp][5] = x1.y; pb[wp][6] = x1.z; pb[wp][7] = x1.w;
        }
        float yv[8];
        {
            const float4 y0 = *reinterpret_cast<const float4 *>(&sm.u.yt[row * kYP + c0]);
            const float4 y1 = *reinterpret_cast<const float4 *>(&sm.u.yt[row * kYP + c0 + 4]);
            yv[0] = y0.x; yv[1] = y0.y; yv[2] = y0.z; yv[3] = y0.w;
            yv[4] = y1.x; yv[5] = y1.y; yv[6] = y1.z; yv[7] = y1.w;
        }
        // bef = exp(G_{r-1}) (blocks before this one), aft = exp(G_n - G_{r-1}) (this block
        // and later), per channel; w is wave-uniform, so these are scalar branches.
        float bef[8], aft[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) { bef[e] = pb[0][e]; aft[e] = pb[3][e]; }
        if (w == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) { bef[e] = 1.f; aft[e] *= pb[2][e] * pb[1][e] * pb[0][e]; }
            if (r16 == 0) {
                *reinterpret_cast<float4 *>(a.gn + ws * kGnElems + c0) = make_float4(aft[0], aft[1], aft[2], aft[3]);
                *reinterpret_cast<float4 *>(a.gn + ws * kGnElems + c0 + 4) = make_float4(aft[4], aft[5], aft[6], aft[7]);
            }
        } else if (w == 1) {
#pragma unroll
            for (int e = 0; e < 8; ++e) aft[e] *= pb[2][e] * pb[1][e];
        } else if (w == 2) {
#pragma unroll
            for (int e = 0; e < 8; ++e) { bef[e] *= pb[1][e]; aft[e] *= pb[2][e]; }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) bef[e] *= pb[1][e] * pb[2][e];
        }
        h8 qg8, kb8, xh, qh;
        s8 xhi, xlo, qhi, qlo, yhi, ylo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int idx = 8 * kk + e;
            qg8[e] = (_Float16)(bef[e] * qv[idx]);            // gamma_i qhat_i
            kgF[kk][e] = (_Float16)(b * bef[e] * kv[idx]);    // b gamma khat
            kb8[e] = (_Float16)(aft[e] * yv[e]);              // exp(G_n - G_j) khat_j
            xh[e] = (_Float16)kv[idx];
            qh[e] = (_Float16)qv[idx];
            short th, tl;
            split_bf16(kv[idx], th, tl); xhi[e] = th; xlo[e] = tl;
            split_bf16(qv[idx], th, tl); qhi[e] = th; qlo[e] = tl;
            split_bf16(yv[e], th, tl); yhi[e] = th; ylo[e] = tl;
        }
        // Qf[w][kk]: lane (r, g) <- Qg[16 w + r][32 kk + 16 half + 4 g + e]   (Sel x Qg^T)
        {
            const f4 lo = mfma16x16x32_f16(sel[0], qg8, f4{0, 0, 0, 0});
            const f4 hi = mfma16x16x32_f16(sel[1], qg8, f4{0, 0, 0, 0});
            store_h8<kStream>(Qf + ((w * 4 + kk) * 64 + lane) * 8, to_h8(lo, hi));
        }
        // Kf[2 kk + half][w / 2]: lane (r, g) <- Kbar[16 w + 4 g + e][32 kk + 16 half + r]   (Kbar x Sel)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const f4 d = mfma16x16x32_f16(kb8, sel[hf], f4{0, 0, 0, 0});
            *reinterpret_cast<h4 *>(Kf + (((2 * kk + hf) * 2 + (w >> 1)) * 64 + lane) * 8 + 4 * (w & 1)) = to_h4(d);
        }
        // Gram tiles, computed transposed: D[j][i], j in block jb, i = this lane's row.
        // Diagonal block: factors span up to exp(+-80), so bf16 hi + lo (three MFMAs).
        akk_d = mfma16x16x32_bf16(yhi, xhi, akk_d);
        akk_d = mfma16x16x32_bf16(yhi, xlo, akk_d);
        akk_d = mfma16x16x32_bf16(ylo, xhi, akk_d);
        aqk_d = mfma16x16x32_bf16(yhi, qhi, aqk_d);
        aqk_d = mfma16x16x32_bf16(yhi, qlo, aqk_d);
        aqk_d = mfma16x16x32_bf16(ylo, qhi, aqk_d);
        // Off-diagonal blocks jb < w: A = [prod_{jb <= w' < w} pblk[w']] * Y_j = exp(G_{r-1} - G_j) khat_j
        // (<= 1, fp16), with r the start of this wave's block.
        float m[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) m[e] = 1.f;
#pragma unroll
        for (int jb = 2; jb >= 0; --jb) {
            if (jb < w) {
#pragma unroll
                for (int e = 0; e < 8; ++e) m[e] *= pb[jb][e];
                const float4 y0 = *reinterpret_cast<const float4 *>(&sm.u.yt[(16 * jb + r16) * kYP + c0]);
                const float4 y1 = *reinterpret_cast<const float4 *>(&sm.u.yt[(16 * jb + r16) * kYP + c0 + 4]);
                h8 yh;
                yh[0] = (_Float16)(y0.x * m[0]); yh[1] = (_Float16)(y0.y * m[1]);
                yh[2] = (_Float16)(y0.z * m[2]); yh[3] = (_Float16)(y0.w * m[3]);
                yh[4] = (_Float16)(y1.x * m[4]); yh[5] = (_Float16)(y1.y * m[5]);
                yh[6] = (_Float16)(y1.z * m[6]); yh[7] = (_Float16)(y1.w * m[7]);
                akk_o[jb] = mfma16x16x32_f16(yh, xh, akk_o[jb]);
                aqk_o[jb] = mfma16x16x32_f16(yh, qh, aqk_o[jb]);
            }
        }
    }
    // Lane holds D[j = 16 jb + 4 cg + e][i = row]: A_kk (b-scaled) to LDS, A_qk to Af.
    {
        f4 dq[4];
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            f4 dk;
            if (jb < w) { dk = akk_o[jb < 3 ? jb : 0]; dq[jb] = aqk_o[jb < 3 ? jb : 0]; }
            else if (jb == w) {
                dk = akk_d; dq[jb] = aqk_d;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int jj = 4 * cg + e;
                    if (!(jj < r16)) dk[e] = 0.f;
                    if (!(jj <= r16)) dq[jb][e] = 0.f;
                }
            } else { dk = f4{0, 0, 0, 0}; dq[jb] = f4{0, 0, 0, 0}; }
            *reinterpret_cast<f4 *>(&sm.L[row * kLP + 16 * jb + 4 * cg]) = dk * b;
        }
        _Float16 *Af = a.Af + ws * kAfElems;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            if (kb == 0 || w >= 2)  // rows 0..31 have no A_qk entries in columns 32..63 (never read)
                store_h8<kStream>(Af + ((w * 2 + kb) * 64 + lane) * 8, to_h8(dq[2 * kb], dq[2 * kb + 1]));
    }
    // ---- P2: invert the diagonal 16x16 blocks of (I + A_kk) -----------------
    // Each wave inverts its own block from the rows it has just written (one
    // wave's LDS accesses execute in order), so this needs no barrier and fills
    // the time the waves with fewer Gram tiles would spend waiting at B2.
    if (cg == 0) {
        // lane r16 = column j of T_ww: forward substitution in fp32.  The strict
        // lower triangle of the block (120 values) is read first, then the
        // substitution runs column by column (x[c] is final when column c is
        // applied), so only one multiply-add per column is on the serial path.
        const int j = r16;
        const float *Lw = sm.L + (16 * w) * kLP + 16 * w;
        float Lt[120];  // L[r][c], c < r, row r at offset r (r - 1) / 2
#pragma unroll
        for (int r = 1; r < 16; ++r)
#pragma unroll
            for (int c = 0; c < r; ++c) Lt[r * (r - 1) / 2 + c] = Lw[r * kLP + c];
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == j) ? 1.f : 0.f;
#pragma unroll
        for (int c = 0; c < 15; ++c)
#pragma unroll
            for (int r = c + 1; r < 16; ++r) x[r] -= Lt[r * (r - 1) / 2 + c] * x[c];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            sm.L[(16 * w + r) * kLP + 16 * w + j] = x[r];
            sm.Th[(16 * w + r) * kTP + 16 * w + j] = (_Float16)x[r];
        }
    }
    // zeros above the diagonal of T
#pragma unroll
    for (int jb = 1; jb < 4; ++jb)
        if (jb > w) *reinterpret_cast<h4 *>(&sm.Th[row * kTP + 16 * jb + 4 * cg]) = h4{0, 0, 0, 0};
    bar();  // B2: L and the diagonal blocks of T complete; the decayed key rows are no longer read

    // ---- P1b: transposed operands of the W / U products into LDS ----------
    //   kg[32 kk + 16 half + r][16 w + 4 g + e] = (b gamma khat)[16 w + 4 g + e][32 kk + 16 half + r]
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int ch = 32 * kk + 16 * hf + r16;
            const f4 dk = mfma16x16x32_f16(kgF[kk], sel[hf], f4{0, 0, 0, 0});
            *reinterpret_cast<h4 *>(&sm.u.t.kg[ch * kTP + 16 * w + 4 * cg]) = to_h4(dk);
            const f4 dv = mfma16x16x32_f16(vbF[kk], sel[hf], f4{0, 0, 0, 0});
            *reinterpret_cast<h4 *>(&sm.u.t.vb[ch * kTP + 16 * w + 4 * cg]) = to_h4(dv);
        }

    // ---- P3: off-diagonal blocks of T, one column block per wave ----------
    switch (w) {
        case 0: offdiag_column<0>(sm, r16, cg); break;
        case 1: offdiag_column<1>(sm, r16, cg); break;
        case 2: offdiag_column<2>(sm, r16, cg); break;
        default: break;
    }
    bar();  // B4: T complete

    // ---- P4: W^T = (b gamma K)^T T^T and U = T (b V) on MFMA ---------------
    {
        const int nkb = w < 2 ? 1 : 2;   // T[i][j] = 0 for j > i
        h8 tf[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            tf[kb] = *reinterpret_cast<const h8 *>(&sm.Th[row * kTP + 32 * kb + 8 * cg]);
        f4 accW[8], accU[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) { accW[t] = f4{0, 0, 0, 0}; accU[t] = f4{0, 0, 0, 0}; }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (kb >= nkb) continue;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const h8 ka = *reinterpret_cast<const h8 *>(&sm.u.t.kg[(16 * t + r16) * kTP + 32 * kb + 8 * cg]);
                accW[t] = mfma16x16x32_f16(ka, tf[kb], accW[t]);
                const h8 vv = *reinterpret_cast<const h8 *>(&sm.u.t.vb[(16 * t + r16) * kTP + 32 * kb + 8 * cg]);
                accU[t] = mfma16x16x32_f16(tf[kb], vv, accU[t]);
            }
        }
        // accW[ct]: W[16 w + r][16 ct + 4 cg + e] -> Wf[w][kb] = -(tiles 2 kb, 2 kb + 1)
        _Float16 *Wf = a.Wf + ws * kWfElems;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
            store_h8<kStream>(Wf + ((w * 4 + kb) * 64 + lane) * 8, to_h8(-accW[2 * kb], -accW[2 * kb + 1]));
        // accU[vt]: U[16 w + 4 cg + e][16 vt + r] -> Uf[vt][w]
        _Float16 *Uf = a.Uf + ws * kUfElems;
#pragma unroll
        for (int vt = 0; vt < 8; ++vt)
            *reinterpret_cast<h4 *>(Uf + ((vt * 4 + w) * 64 + lane) * 4) = to_h4(accU[vt]);
    }
}

}  // namespace intra
}  // namespace kda
