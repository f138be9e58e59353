// kda_intra.hip -- intra-chunk kernel of the KDA forward pass (gfx950).
//
// One 256-thread workgroup per (64-token chunk, head).  It fuses the in-kernel
// activations the forward call applies (q/k L2 norm, beta sigmoid, the gate
// from g / A_log / dt_bias clamped at lower_bound; "作为 FLA 后端的用法",
// zuobiaodaohang.com FlashKDA page) with the chunk-local algebra of the
// chunk-parallel delta rule:
//
//   gamma_i = exp(G_i), G_i = sum_{t<=i} a_t              (per channel, within the chunk)
//   A_kk[i,j] = b_i sum_d khat_i[d] khat_j[d] exp(G_i[d]-G_j[d]),  j < i
//   A_qk[i,j] =     sum_d qhat_i[d] khat_j[d] exp(G_i[d]-G_j[d]),  j <= i
//   T = (I + A_kk)^-1,  W = T Diag(b) (gamma * Khat),  U = T Diag(b) V
//   Kbar_j = exp(G_n - G_j) * khat_j,  Qg_i = gamma_i * qhat_i
//
// (the WY/UT representation of products of Householder-like factors, as used
// for delta-rule attention by Yang et al., "Parallelizing Linear Transformers
// with the Delta Rule over Sequence Length", extended here to a per-channel
// decay).  The state chain kernel consumes W, U, Kbar, Qg, A_qk, exp(G_n).
//
// Decay factors exp(G_i - G_j) are never formed as exp(G_i) * exp(-G_j) over a
// whole chunk (that overflows): within each 16-row block r..r+15 the kernel
// keeps P_i = exp(G_i - G_{r-1}) (a product of at most 16 factors >= exp(-5),
// so >= exp(-80) > FLT_MIN), and off-diagonal 16x16 blocks use the row
// block's start as the reference so that both MFMA factors are <= 1.  That is
// what the lower bound of -5 on the log-decay buys.
//
// Matrix products run on MFMA with fp16 operands and fp32 accumulation; the
// diagonal 16x16 blocks of the two Gram matrices, whose factors span up to
// exp(+-80), use bf16 hi+lo splits (three bf16 MFMAs); the triangular inverse
// is done in fp32 (diagonal blocks) and split-fp16 MFMA (off-diagonal blocks).
#include "kda_common.h"

using namespace kda;

namespace {

constexpr int kThreads = 256;

struct __align__(16) IntraSmem {
    float yt[48 * 128];      // rows of blocks 0..2: exp(G_e - G_j) * khat_j, e = block end of the row
    float L[64 * 64];        // A_kk (b-scaled, strictly lower), overwritten in place by T
    _Float16 kgT[128 * 64];  // (b * gamma * khat)^T, [channel][token]
    _Float16 vbT[128 * 64];  // (b * v)^T,            [value column][token]
    float pblk[4 * 128];     // per 16-row block: product of the block's decays, per channel
};

__device__ __forceinline__ h4 to_h4(const f4 &x) {
    h4 r;
    r[0] = (_Float16)x[0]; r[1] = (_Float16)x[1]; r[2] = (_Float16)x[2]; r[3] = (_Float16)x[3];
    return r;
}

// fp16 hi + lo split of four floats.
__device__ __forceinline__ void split_h4(const float *x, h4 &hi, h4 &lo) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        _Float16 h = (_Float16)x[e];
        hi[e] = h;
        lo[e] = (_Float16)(x[e] - (float)h);
    }
}

__device__ __forceinline__ f4 mfma_split16(const h4 &ah, const h4 &al, const h4 &bh, const h4 &bl, f4 c) {
    c = mfma16x16x16_f16(ah, bh, c);
    c = mfma16x16x16_f16(ah, bl, c);
    c = mfma16x16x16_f16(al, bh, c);
    return c;
}

// Gram tiles of row block W, computed transposed (D[j][i], j in block jb,
// i = this wave's rows): A_kk (b-scaled, strictly lower) to LDS in fp32 and
// A_qk (lower incl. diagonal) to global in fp16.  Blocks above the diagonal
// are written as zeros.
template <int W>
__device__ __forceinline__ void gram_tiles(IntraSmem &sm, const float *kv, const float *qv, const float *yd,
                                           float b, int row, int r16, int cg, _Float16 *Aqk) {
    f4 akk_o[W > 0 ? W : 1], aqk_o[W > 0 ? W : 1];
    f4 akk_d = f4{0, 0, 0, 0}, aqk_d = f4{0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < (W > 0 ? W : 1); ++t) { akk_o[t] = f4{0, 0, 0, 0}; aqk_o[t] = f4{0, 0, 0, 0}; }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int c0 = 32 * kk + 8 * cg;
        s8 xhi, xlo, qhi, qlo, ydhi, ydlo;
        h8 xh, qh;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int idx = 8 * kk + e;
            short th, tl;
            split_bf16(kv[idx], th, tl); xhi[e] = th; xlo[e] = tl;
            split_bf16(qv[idx], th, tl); qhi[e] = th; qlo[e] = tl;
            split_bf16(yd[idx], th, tl); ydhi[e] = th; ydlo[e] = tl;
            xh[e] = (_Float16)kv[idx];
            qh[e] = (_Float16)qv[idx];
        }
        // diagonal block: factors span up to exp(+-80), so bf16 hi+lo (3 MFMAs)
        akk_d = mfma16x16x32_bf16(ydhi, xhi, akk_d);
        akk_d = mfma16x16x32_bf16(ydhi, xlo, akk_d);
        akk_d = mfma16x16x32_bf16(ydlo, xhi, akk_d);
        aqk_d = mfma16x16x32_bf16(ydhi, qhi, aqk_d);
        aqk_d = mfma16x16x32_bf16(ydhi, qlo, aqk_d);
        aqk_d = mfma16x16x32_bf16(ydlo, qhi, aqk_d);
        if constexpr (W > 0) {
            // off-diagonal blocks jb < W: A = [prod_{jb < w' < W} pblk[w']] * yt_j  (<= 1, fp16)
            float m[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) m[e] = 1.f;
#pragma unroll
            for (int jb = W - 1; jb >= 0; --jb) {
                if (jb < W - 1) {
                    const float4 p0 = *reinterpret_cast<const float4 *>(&sm.pblk[(jb + 1) * 128 + c0]);
                    const float4 p1 = *reinterpret_cast<const float4 *>(&sm.pblk[(jb + 1) * 128 + c0 + 4]);
                    m[0] *= p0.x; m[1] *= p0.y; m[2] *= p0.z; m[3] *= p0.w;
                    m[4] *= p1.x; m[5] *= p1.y; m[6] *= p1.z; m[7] *= p1.w;
                }
                const float4 y0 = *reinterpret_cast<const float4 *>(&sm.yt[(16 * jb + r16) * 128 + c0]);
                const float4 y1 = *reinterpret_cast<const float4 *>(&sm.yt[(16 * jb + r16) * 128 + c0 + 4]);
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
    // Lane holds D[j = 16 jb + 4 cg + e][i = row].
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
        f4 dk, dq;
        if (jb < W) { dk = akk_o[jb < W ? jb : 0]; dq = aqk_o[jb < W ? jb : 0]; }
        else if (jb == W) {
            dk = akk_d; dq = aqk_d;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int jj = 4 * cg + e;
                if (!(jj < r16)) dk[e] = 0.f;
                if (!(jj <= r16)) dq[e] = 0.f;
            }
        } else { dk = f4{0, 0, 0, 0}; dq = f4{0, 0, 0, 0}; }
        dk = dk * b;
        *reinterpret_cast<f4 *>(&sm.L[row * 64 + 16 * jb + 4 * cg]) = dk;
        h4 qq;
        qq[0] = (_Float16)dq[0]; qq[1] = (_Float16)dq[1]; qq[2] = (_Float16)dq[2]; qq[3] = (_Float16)dq[3];
        *reinterpret_cast<h4 *>(Aqk + row * 64 + 16 * jb + 4 * cg) = qq;
    }
}

__global__ __launch_bounds__(kThreads, 2) void kda_intra_kernel(IntraArgs a) {
    __shared__ IntraSmem sm;

    const int64_t slot = blockIdx.x;
    const int64_t h = blockIdx.y;
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

    const int tid = threadIdx.x;
    const int w = tid >> 6;          // wave = 16-row block
    const int lane = tid & 63;
    const int r16 = lane & 15;       // row within the block
    const int cg = lane >> 4;        // 8-channel group within each 32-channel step
    const int row = 16 * w + r16;
    const bool valid = row < L;

    const int64_t ws = slot * H + h;  // workspace index of this (chunk, head)
    _Float16 *Wn = a.Wn + ws * kWnElems;
    _Float16 *Qg = a.Qg + ws * kQgElems;
    _Float16 *Kbt = a.Kbt + ws * kKbtElems;
    _Float16 *Ut = a.Ut + ws * kUtElems;
    _Float16 *Aqk = a.Aqk + ws * kAqkElems;
    float *gn = a.gn + ws * kGnElems;

    // ---- P0: load, normalise, gate, block-local decay products ------------
    // Lane owns row `row`, channels ch(kk, e) = 32 kk + 8 cg + e.
    float qv[32], kv[32];
    uint4 graw[4], vraw[4];
    {
        const int64_t base = ((t0 + row) * H + h) * kK;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int c0 = 32 * kk + 8 * cg;
            uint4 qr = make_uint4(0, 0, 0, 0), kr = qr, gr = qr, vr = qr;
            if (valid) {
                qr = *reinterpret_cast<const uint4 *>(a.q + base + c0);
                kr = *reinterpret_cast<const uint4 *>(a.k + base + c0);
                gr = *reinterpret_cast<const uint4 *>(a.g + base + c0);
                vr = *reinterpret_cast<const uint4 *>(a.v + base + c0);
            }
            unpack_bf16x8(qr, qv + 8 * kk);
            unpack_bf16x8(kr, kv + 8 * kk);
            graw[kk] = gr;
            vraw[kk] = vr;
        }
    }
    float ssq = 0.f, ssk = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) { ssq += qv[e] * qv[e]; ssk += kv[e] * kv[e]; }
    ssq += __shfl_xor(ssq, 16); ssq += __shfl_xor(ssq, 32);
    ssk += __shfl_xor(ssk, 16); ssk += __shfl_xor(ssk, 32);
    const float rq = fast_rsqrt(ssq + 1e-6f);
    const float rk = fast_rsqrt(ssk + 1e-6f);
    float b = 0.f;
    if (valid) b = fast_rcp(1.0f + fast_exp(-bf16_bits_to_f32(a.beta[(t0 + row) * H + h])));

    // gate: d = exp(max(lb, -exp(A_log) softplus(g + dt_bias))), then the
    // inclusive product over the block's rows: P_i = exp(G_i - G_{r-1}).
    float P[32];
    {
        const float Aexp = fast_exp(a.A_log[h]);
        const float lb = a.lower_bound;
        const float *dtb = a.dt_bias + h * kK;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int c0 = 32 * kk + 8 * cg;
            const float4 d0 = *reinterpret_cast<const float4 *>(dtb + c0);
            const float4 d1 = *reinterpret_cast<const float4 *>(dtb + c0 + 4);
            const float db[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
            float gf[8];
            unpack_bf16x8(graw[kk], gf);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = gf[e] + db[e];
                // softplus(x) = max(x,0) + log1p(u), u = exp(-|x|) in (0, 1]; a short
                // series for small u keeps log1p accurate where 1 + u would round
                const float u = fast_exp(-fabsf(x));
                const float small = u * (1.0f - u * (0.5f - u * (1.0f / 3.0f)));
                const float sp = fmaxf(x, 0.f) + (u < (1.0f / 128.0f) ? small : fast_log(1.0f + u));
                const float lg = fmaxf(lb, -Aexp * sp);
                P[8 * kk + e] = valid ? fast_exp(lg) : 1.0f;
            }
        }
    }
#pragma unroll
    for (int s = 1; s < 16; s <<= 1) {
#pragma unroll
        for (int e = 0; e < 32; ++e) P[e] *= dpp_row_shr(P[e], 1.0f, s);
    }
    // yd = exp(G_{r-1} - G_j) khat_j (>= khat; used by the diagonal blocks), and
    // exp(G_e - G_j) khat_j = pe * yd with e the block end and pe the block total
    float yd[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        const float pe = dpp_row_bcast15(P[e]);
        const float kh = kv[e] * rk;
        yd[e] = kh * fast_rcp(P[e]);
        kv[e] = kh * P[e];         // X_i = exp(G_i - G_{r-1}) khat_i
        qv[e] = qv[e] * rq * P[e]; // Q'_i = exp(G_i - G_{r-1}) qhat_i
        P[e] = pe;
    }
    if (w < 3) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int i0 = 8 * kk;
            float4 *dst = reinterpret_cast<float4 *>(&sm.yt[row * 128 + 32 * kk + 8 * cg]);
            dst[0] = make_float4(P[i0 + 0] * yd[i0 + 0], P[i0 + 1] * yd[i0 + 1], P[i0 + 2] * yd[i0 + 2], P[i0 + 3] * yd[i0 + 3]);
            dst[1] = make_float4(P[i0 + 4] * yd[i0 + 4], P[i0 + 5] * yd[i0 + 5], P[i0 + 6] * yd[i0 + 6], P[i0 + 7] * yd[i0 + 7]);
        }
    }
    if (r16 == 15) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            float4 *dst = reinterpret_cast<float4 *>(&sm.pblk[w * 128 + 32 * kk + 8 * cg]);
            dst[0] = make_float4(P[8 * kk + 0], P[8 * kk + 1], P[8 * kk + 2], P[8 * kk + 3]);
            dst[1] = make_float4(P[8 * kk + 4], P[8 * kk + 5], P[8 * kk + 6], P[8 * kk + 7]);
        }
    }
    lds_barrier();  // B1

    // ---- P1: cross-block decays, outputs that need only gamma, Gram tiles --
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
        float vf[8];
        unpack_bf16x8(vraw[kk], vf);
        h8 qg8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int ch = c0 + e;
            const float gb = (w > 0 ? pb[0][e] : 1.f) * (w > 1 ? pb[1][e] : 1.f) * (w > 2 ? pb[2][e] : 1.f);
            const float ga = (w < 1 ? pb[1][e] : 1.f) * (w < 2 ? pb[2][e] : 1.f) * (w < 3 ? pb[3][e] : 1.f);
            const int idx = 8 * kk + e;
            qg8[e] = (_Float16)(gb * qv[idx]);                        // gamma_i qhat_i
            sm.kgT[ch * 64 + row] = (_Float16)(b * gb * kv[idx]);     // b gamma khat
            sm.vbT[ch * 64 + row] = (_Float16)(b * vf[e]);            // b v
            Kbt[ch * 64 + row] = (_Float16)(ga * (P[idx] * yd[idx]));  // exp(G_n - G_j) khat_j, transposed
        }
        if (w == 0 && r16 == 0) {
            *reinterpret_cast<float4 *>(gn + c0) = make_float4(
                pb[0][0] * pb[1][0] * pb[2][0] * pb[3][0], pb[0][1] * pb[1][1] * pb[2][1] * pb[3][1],
                pb[0][2] * pb[1][2] * pb[2][2] * pb[3][2], pb[0][3] * pb[1][3] * pb[2][3] * pb[3][3]);
            *reinterpret_cast<float4 *>(gn + c0 + 4) = make_float4(
                pb[0][4] * pb[1][4] * pb[2][4] * pb[3][4], pb[0][5] * pb[1][5] * pb[2][5] * pb[3][5],
                pb[0][6] * pb[1][6] * pb[2][6] * pb[3][6], pb[0][7] * pb[1][7] * pb[2][7] * pb[3][7]);
        }
        *reinterpret_cast<h8 *>(Qg + row * kK + c0) = qg8;
    }

    switch (w) {
        case 0: gram_tiles<0>(sm, kv, qv, yd, b, row, r16, cg, Aqk); break;
        case 1: gram_tiles<1>(sm, kv, qv, yd, b, row, r16, cg, Aqk); break;
        case 2: gram_tiles<2>(sm, kv, qv, yd, b, row, r16, cg, Aqk); break;
        default: gram_tiles<3>(sm, kv, qv, yd, b, row, r16, cg, Aqk); break;
    }
    lds_barrier();  // B2: L complete, yt free, kgT/vbT complete

    // ---- P2: invert the diagonal 16x16 blocks of (I + A_kk) -----------------
    if (cg == 0) {
        // lane r16 = column j of T_ww; left-looking forward substitution in fp32
        const int j = r16;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == j) ? 1.f : 0.f;
        const float *Lw = sm.L + (16 * w) * 64 + 16 * w;
#pragma unroll
        for (int r = 1; r < 16; ++r) {
            float acc = x[r];
#pragma unroll
            for (int kq = 0; kq < r; ++kq) acc -= Lw[r * 64 + kq] * x[kq];
            x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.L[(16 * w + r) * 64 + 16 * w + j] = x[r];
    }
    lds_barrier();  // B3

    // ---- P3: off-diagonal blocks of T, row block by row block -------------
    //   T_ij = -T_ii * sum_{k=j}^{i-1} L_ik T_kj  (16x16 blocks, split-fp16 MFMA)
#pragma unroll
    for (int ib = 1; ib < 4; ++ib) {
        f4 tij = f4{0, 0, 0, 0};
        if (w < ib) {
            const int jb = w;
            f4 R = f4{0, 0, 0, 0};
            for (int kb = jb; kb < ib; ++kb) {
                float av[4], bv[4];
                const float4 la = *reinterpret_cast<const float4 *>(&sm.L[(16 * ib + r16) * 64 + 16 * kb + 4 * cg]);
                av[0] = la.x; av[1] = la.y; av[2] = la.z; av[3] = la.w;
#pragma unroll
                for (int e = 0; e < 4; ++e) bv[e] = sm.L[(16 * kb + 4 * cg + e) * 64 + 16 * jb + r16];
                h4 ah, al, bh, bl;
                split_h4(av, ah, al);
                split_h4(bv, bh, bl);
                R = mfma_split16(ah, al, bh, bl, R);
            }
            float av[4], bv[4];
            const float4 ta = *reinterpret_cast<const float4 *>(&sm.L[(16 * ib + r16) * 64 + 16 * ib + 4 * cg]);
            av[0] = ta.x; av[1] = ta.y; av[2] = ta.z; av[3] = ta.w;
            bv[0] = R[0]; bv[1] = R[1]; bv[2] = R[2]; bv[3] = R[3];
            h4 ah, al, bh, bl;
            split_h4(av, ah, al);
            split_h4(bv, bh, bl);
            tij = mfma_split16(ah, al, bh, bl, tij);
        }
        lds_barrier();
        if (w < ib) {
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.L[(16 * ib + 4 * cg + e) * 64 + 16 * w + r16] = -tij[e];
        }
        lds_barrier();
    }

    // ---- P4: W^T = (Kg)^T T^T and U = T Vb on MFMA --------------------------
    f4 accW[4][2], accU[4][2];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int t = 0; t < 2; ++t) { accW[ib][t] = f4{0, 0, 0, 0}; accU[ib][t] = f4{0, 0, 0, 0}; }
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            if (ks == 1 && ib < 2) continue;
            // T[i = 16 ib + r16][j = 32 ks + 8 cg + e]
            const float *tp = &sm.L[(16 * ib + r16) * 64 + 32 * ks + 8 * cg];
            const float4 t0v = *reinterpret_cast<const float4 *>(tp);
            const float4 t1v = *reinterpret_cast<const float4 *>(tp + 4);
            h8 tf;
            tf[0] = (_Float16)t0v.x; tf[1] = (_Float16)t0v.y; tf[2] = (_Float16)t0v.z; tf[3] = (_Float16)t0v.w;
            tf[4] = (_Float16)t1v.x; tf[5] = (_Float16)t1v.y; tf[6] = (_Float16)t1v.z; tf[7] = (_Float16)t1v.w;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int rt = 2 * w + t;  // channel tile (W^T rows) and value-column tile (U columns)
                const h8 ka = *reinterpret_cast<const h8 *>(&sm.kgT[(16 * rt + r16) * 64 + 32 * ks + 8 * cg]);
                accW[ib][t] = mfma16x16x32_f16(ka, tf, accW[ib][t]);
                const h8 vb = *reinterpret_cast<const h8 *>(&sm.vbT[(16 * rt + r16) * 64 + 32 * ks + 8 * cg]);
                accU[ib][t] = mfma16x16x32_f16(tf, vb, accU[ib][t]);
            }
        }
    }
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int rt = 2 * w + t;
            // accW: D[c = 16 rt + 4 cg + e][i = 16 ib + r16]  ->  Wn[i][c..c+3] = -W
            const f4 wv = -accW[ib][t];
            *reinterpret_cast<h4 *>(Wn + (16 * ib + r16) * kK + 16 * rt + 4 * cg) = to_h4(wv);
            // accU: D[i = 16 ib + 4 cg + e][v = 16 rt + r16]  ->  Ut[v][i..i+3]
            *reinterpret_cast<h4 *>(Ut + (16 * rt + r16) * kChunk + 16 * ib + 4 * cg) = to_h4(accU[ib][t]);
        }
    }
}

}  // namespace

hipError_t kda_launch_intra(const IntraArgs &a, int64_t slots, hipStream_t s) {
    if (slots <= 0) return hipSuccess;
    dim3 grid((unsigned)slots, (unsigned)a.H);
    hipLaunchKernelGGL(kda_intra_kernel, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}
