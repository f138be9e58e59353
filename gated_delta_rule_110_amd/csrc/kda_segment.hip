// kda_segment.hip -- split state chains: segment table and the scan over segments (gfx950).
//
// A long sequence's state chain is serial over its chunks, and one sequence
// with few heads gives the chain kernel only 8 workgroups per head.  Each
// chunk maps the entering state affinely, S -> (Diag(exp(G_n)) - Kbar^T W) S
// + Kbar^T U (the chunk form of the KDA recurrence; "¿Qué es la atención Kimi
// Delta…", 7minutos.es, and the WY/UT chunking of delta-rule attention by Yang
// et al., "Parallelizing Linear Transformers with the Delta Rule over Sequence
// Length"), and affine maps compose.  So the chunks of a sequence are cut into
// segments, and the forward pass runs in three steps:
//
//   1. the chain kernel in map mode gives every segment its map S -> M S + N
//      (all segments at once: M from S = I with U = 0, N from S = 0);
//   2. this file's scan composes them in order, S_{s+1} = M_s S_s + N_s,
//      starting from the initial state, which gives the state entering every
//      segment and the final state;
//   3. the chain kernel runs every segment from its entering state as if the
//      segments were separate packed sequences, writing the outputs.
//
// Segments start on chunk boundaries, so the chunk slots the intra-chunk
// kernel wrote are those of the packed view built here.
#include "kda_common.h"

using namespace kda;

namespace {

constexpr int kThreads = 256;
constexpr int kCols = 16;    // state columns per workgroup
constexpr int kSP = 132;     // pitch (floats) of a column of the state slice in LDS

// The segments of every batch row as packed sequences: segment s of row b is
// packed sequence b * segs + s, starting at chunk s * segc of the row.
__global__ __launch_bounds__(kThreads) void kda_seg_table_kernel(int64_t B, int64_t T, int64_t segs,
                                                                 int64_t segc, int64_t *cu, int32_t *off) {
    const int64_t nc = (T + kChunk - 1) / kChunk;
    const int64_t n = B * segs;
    for (int64_t i = threadIdx.x; i <= n; i += kThreads) {
        int64_t c, t;
        if (i == n) {
            c = B * nc;
            t = B * T;
        } else {
            const int64_t b = i / segs, s = i - b * segs;
            const int64_t cs = s * segc < nc ? s * segc : nc;
            c = b * nc + cs;
            t = b * T + (cs * kChunk < T ? cs * kChunk : T);
        }
        cu[i] = t;
        off[i] = (int32_t)c;
    }
}

// One workgroup per (16-column block, batch row and head).  The slice S[:, cols]
// (128 x 16 fp32) lives in LDS, transposed, double-buffered; each step is the
// fp32 product M_s S (128 x 128 times 128 x 16) on the matrix cores plus N_s.
// Wave w computes row tile w.  The 16x16x4 fp32 MFMA sums over the four
// 16-lane groups; lane group q of product j takes k = 16 kq + 4 q + j in both
// operands, so one 16-byte load per lane feeds four products.  The next
// segment's M and N rows are loaded while the current product runs: the
// scan is a chain of dependent steps, and each step's loads would otherwise
// be exposed.
// kRev is the gradient's pass (ScanArgs::reverse): segments last to first and
// the product M_s^T D, whose A operand is read down the columns of M_s (four
// 64-byte row pieces per kq instead of one 16-byte load).
constexpr int kScanThreads = 512;

template <bool kRev>
__device__ __forceinline__ void seg_scan(const ScanArgs &a) {
    __shared__ float st[2][kCols * kSP];  // [buffer][column * kSP + row]

    const int64_t bh = blockIdx.x;  // on x: a grid's y extent is small
    const int vb = blockIdx.y;
    const int64_t b = bh / a.H, h = bh - b * a.H;
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, r = lane & 15, q = lane >> 4;
    constexpr int64_t KV = (int64_t)kK * kV;
    const int64_t col0 = (int64_t)kCols * vb;
    auto seg_index = [&](int64_t s) { return (b * a.segs + s) * a.H + h; };
    // the i-th step works on segment first + dir * i
    const int64_t first = kRev ? a.segs - 1 : 0, dir = kRev ? -1 : 1;

    {   // the starting value (h0[b, h] or zeros): thread t holds column t % 16, rows 4 (t / 16) .. + 3;
        // forward it enters segment 0, reverse it leaves the last segment
        const int c = tid & 15, r0 = 4 * (tid >> 4);
        const int64_t src = bh * KV + col0 + c;
        float *dst = a.sin + seg_index(first) * KV + col0 + c;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = r0 + i;
            float v = 0.f;
            if (a.h0) v = a.h0_bf16 ? bf16_bits_to_f32(static_cast<const uint16_t *>(a.h0)[src + row * kV])
                                    : static_cast<const float *>(a.h0)[src + row * kV];
            st[0][c * kSP + row] = v;
            dst[row * kV] = v;
        }
    }

    // this lane's operands of segment s: the A rows 16 w + r, k = 16 kq + 4 q .. + 3
    // (M_s, or M_s^T), and N[16 w + 4 q + e][col0 + r]
    f4 am[8], an;
    auto load = [&](int64_t s) {
        const float *M = a.mapM + seg_index(s) * KV;
#pragma unroll
        for (int kq = 0; kq < 8; ++kq) {
            if constexpr (kRev) {
#pragma unroll
                for (int j = 0; j < 4; ++j) am[kq][j] = M[(16 * kq + 4 * q + j) * kK + 16 * w + r];
            } else {
                am[kq] = *reinterpret_cast<const f4 *>(M + (16 * w + r) * kK + 16 * kq + 4 * q);
            }
        }
        const float *N = a.mapN + seg_index(s) * KV + (16 * w + 4 * q) * kV + col0 + r;
#pragma unroll
        for (int e = 0; e < 4; ++e) an[e] = N[e * kV];
    };
    load(first);
    __syncthreads();

    for (int64_t i = 0; i < a.segs; ++i) {
        const int64_t s = first + dir * i;
        const int p = (int)(i & 1);
        f4 m[8], n = an;
#pragma unroll
        for (int kq = 0; kq < 8; ++kq) m[kq] = am[kq];
        if (i + 1 < a.segs) load(s + dir);
        f4 acc = f4{0, 0, 0, 0};
#pragma unroll
        for (int kq = 0; kq < 8; ++kq) {
            const f4 bs = *reinterpret_cast<const f4 *>(&st[p][r * kSP + 16 * kq + 4 * q]);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(m[kq][j], bs[j], acc, 0, 0, 0);
        }
        // lane (r, q) holds rows 16 w + 4 q + e of column r
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * w + 4 * q + e;
            const float v = acc[e] + n[e];
            st[p ^ 1][r * kSP + row] = v;
            if (i + 1 < a.segs) {
                a.sin[seg_index(s + dir) * KV + row * kV + col0 + r] = v;
            } else if (a.ht) {
                const int64_t idx = bh * KV + row * kV + col0 + r;
                if (a.ht_bf16) static_cast<uint16_t *>(a.ht)[idx] = f32_to_bf16_bits(v);
                else static_cast<float *>(a.ht)[idx] = v;
            }
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(kScanThreads) void kda_seg_scan_kernel(ScanArgs a) { seg_scan<false>(a); }
__global__ __launch_bounds__(kScanThreads) void kda_seg_scan_rev_kernel(ScanArgs a) { seg_scan<true>(a); }

}  // namespace

hipError_t kda_launch_seg_table(int64_t B, int64_t T, int64_t segs, int64_t segc, int64_t *cu, int32_t *off,
                                hipStream_t s) {
    hipLaunchKernelGGL(kda_seg_table_kernel, dim3(1), dim3(kThreads), 0, s, B, T, segs, segc, cu, off);
    return hipGetLastError();
}

hipError_t kda_launch_seg_scan(const ScanArgs &a, hipStream_t s) {
    const int64_t bh = a.B * a.H;
    if (bh <= 0 || a.segs <= 0) return hipSuccess;
    if (a.reverse)
        hipLaunchKernelGGL(kda_seg_scan_rev_kernel, dim3((unsigned)bh, (unsigned)(kV / kCols)), dim3(kScanThreads), 0,
                           s, a);
    else
        hipLaunchKernelGGL(kda_seg_scan_kernel, dim3((unsigned)bh, (unsigned)(kV / kCols)), dim3(kScanThreads), 0,
                           s, a);
    return hipGetLastError();
}
