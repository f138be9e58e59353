// kda_decode.hip -- one recurrent KDA step per sequence (gfx950).
//
// The recurrent form of the method processes one token per step, which is
// how generation proceeds ("¿Qué es la atención Kimi Delta y por qué es
// importante?", 7minutos.es).  For every (sequence n, head h), with the K x V
// state S read from initial_state (or zero):
//
//   S' = (I - b k k^T) Diag(exp(a)) S + b k v^T,    o = scale * S'^T q
//
// with the same in-kernel L2 norms, sigmoid and gate as the chunked forward.
// Writing D = Diag(exp(a)) S, the step needs two reductions over the K rows
// of D -- D^T k and D^T q -- after which
//
//   u = b (v - D^T k),   S' = D + k u^T,   o = scale (D^T q + u (k . q)).
//
// So the state is read once, decayed in registers, reduced, and written once:
// the step is bound by the state's HBM traffic (2 x 64 KiB per head in fp32).
//
// One 256-thread workgroup per (sequence, head), or per (sequence, head, slice
// of 64 or 32 value columns) for small batches.  With one slice, thread (wave
// w, lane l) holds rows 32 w .. 32 w + 31 and columns 2 l, 2 l + 1 of S, so each
// row is one coalesced 512-byte (fp32) or 256-byte (bf16) access per wave.
#include "kda_common.h"

using namespace kda;

namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
typedef float f2 __attribute__((ext_vector_type(2)));

// States of at least this many bytes are read and written with non-temporal
// hints: they cannot stay in the 256 MiB Infinity Cache between steps anyway,
// and streaming them past it measured 11% faster (N = 256 and 1024 sequences
// of 32 heads).  Smaller states are cached, so that a state updated in place
// step after step is partly served from the Infinity Cache (N = 64: 41 us
// cached against 47 us streamed).
constexpr int64_t kStreamStateBytes = 256ll << 20;

// Small batches spread each head over 4 column slices while that makes at
// most kSplitWorkgroups workgroups, then over 2 slices up to twice that
// (graph-replayed steps at 32 heads: N = 1 5.9 -> 3.5 us, N = 4 6.8 -> 4.8 us
// with 4 slices, N = 16 11.2 -> 10.4 us with 2; from N = 32 one slice is best).
constexpr int64_t kSplitWorkgroups = 512;

template <bool kNT, typename T>
__device__ __forceinline__ T state_load(const T *p) {
    if constexpr (kNT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool kNT, typename T>
__device__ __forceinline__ void state_store(T *p, T v) {
    if constexpr (kNT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

struct __align__(16) DecodeSmem {
    float kh[kK];          // normalised key
    float qh[kK];          // normalised query
    float dec[kK];         // exp(a), per channel
    float part[8 * kV];    // per-row-group partial sums of D^T k and D^T q, [group][column][2]
    float scal[4];         // b, k.q
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
    return x;
}

// One workgroup per (sequence, head, slice of kV / kS value columns).  The
// state's columns are independent through the whole step (D^T k, u, the
// update and D^T q are all per column), so a head can be spread over kS
// workgroups, each recomputing the per-token vectors; small batches then use
// more of the GPU.  Thread t holds the column pair p = t % kPairs of its slice
// and the rows kRows rg .. kRows rg + kRows - 1, rg = t / kPairs.
template <bool kNT, int kS>
__device__ __forceinline__ void decode_body(const DecodeArgs &a) {
    constexpr int kCols = kV / kS;              // value columns of this workgroup
    constexpr int kPairs = kCols / 2;           // threads per row group
    constexpr int kGroups = kThreads / kPairs;  // row groups
    constexpr int kRows = kK / kGroups;         // rows per thread
    static_assert(kGroups * kCols * 2 <= 8 * kV, "partial sums must fit");
    __shared__ DecodeSmem sm;
    const int64_t local = blockIdx.x / kS;
    const int slice = (int)(blockIdx.x - local * kS);
    const int64_t unit = a.unit_base + local;
    const int64_t n = unit / a.H, h = unit - (unit / a.H) * a.H;
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63;
    const int p = tid % kPairs, rg = tid / kPairs;
    const int cl = 2 * p;
    const int col = kCols * slice + cl;
    const int64_t row = n * a.H + h;
    // ---- state loads first: the per-token vector work below runs while they
    // are in flight (otherwise the state's HBM latency follows the vectors') --
    const int64_t sbase = (n * a.H + h) * (int64_t)kK * kV + col;
    float D[kRows][2];
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        const int c = kRows * rg + i;
        const int64_t idx = sbase + (int64_t)c * kV;
        float s0 = 0.f, s1 = 0.f;
        if (a.h0) {
            if (a.h0_bf16) {
                const uint32_t pr = state_load<kNT>(reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint16_t *>(a.h0) + idx));
                s0 = bf16_bits_to_f32(pr & 0xffffu);
                s1 = bf16_bits_to_f32(pr >> 16);
            } else {
                const f2 pr = state_load<kNT>(reinterpret_cast<const f2 *>(reinterpret_cast<const float *>(a.h0) + idx));
                s0 = pr[0];
                s1 = pr[1];
            }
        }
        D[i][0] = s0;
        D[i][1] = s1;
    }
    // ---- per-token vectors: L2 norms (waves 0, 1), gate (waves 2, 3) ------
    if (w < 2) {
        const uint16_t *src = (w == 0 ? a.k : a.q) + row * kK;
        const uint32_t pair = *reinterpret_cast<const uint32_t *>(src + 2 * lane);
        const float x0 = bf16_bits_to_f32(pair & 0xffffu), x1 = bf16_bits_to_f32(pair >> 16);
        const float r = fast_rsqrt(wave_sum(x0 * x0 + x1 * x1) + 1e-6f);
        float *dst = w == 0 ? sm.kh : sm.qh;
        dst[2 * lane] = x0 * r;
        dst[2 * lane + 1] = x1 * r;
    } else {
        const int c = 64 * (w - 2) + lane;
        const float x = bf16_bits_to_f32(a.g[row * kK + c]) + a.dt_bias[h * kK + c];
        const float nA = -fast_exp(a.A_log[h]);
        const float l2 = gate_log2(x, nA, a.lower_bound * kLog2e);
        sm.dec[c] = __builtin_amdgcn_exp2f(l2);
        if (w == 2 && lane == 0) sm.scal[0] = fast_rcp(1.0f + fast_exp(-bf16_bits_to_f32(a.beta[row])));
    }
    __syncthreads();
    if (w == 0) {
        const float kq = wave_sum(sm.kh[2 * lane] * sm.qh[2 * lane] + sm.kh[2 * lane + 1] * sm.qh[2 * lane + 1]);
        if (lane == 0) sm.scal[1] = kq;
    }
    // ---- state pass: D = Diag(exp(a)) S, partial D^T k and D^T q ----------
    float pk0 = 0.f, pk1 = 0.f, pq0 = 0.f, pq1 = 0.f;
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        const int c = kRows * rg + i;
        const float d = sm.dec[c], kc = sm.kh[c], qc = sm.qh[c];
        D[i][0] *= d;
        D[i][1] *= d;
        pk0 += D[i][0] * kc; pk1 += D[i][1] * kc;
        pq0 += D[i][0] * qc; pq1 += D[i][1] * qc;
    }
    float *part = sm.part;
    *reinterpret_cast<float2 *>(&part[(rg * kCols + cl) * 2]) = make_float2(pk0, pq0);
    *reinterpret_cast<float2 *>(&part[(rg * kCols + cl + 1) * 2]) = make_float2(pk1, pq1);
    __syncthreads();
    // ---- u = b (v - D^T k) for this thread's two columns; output by row group 0
    float u[2], dq[2];
    const float b = sm.scal[0];
    const uint32_t vpair = *reinterpret_cast<const uint32_t *>(a.v + row * kV + col);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        float dk = 0.f;
        dq[j] = 0.f;
#pragma unroll
        for (int gq = 0; gq < kGroups; ++gq) {
            dk += part[(gq * kCols + cl + j) * 2];
            dq[j] += part[(gq * kCols + cl + j) * 2 + 1];
        }
        const float vj = bf16_bits_to_f32(j == 0 ? (vpair & 0xffffu) : (vpair >> 16));
        u[j] = b * (vj - dk);
    }
    if (rg == 0) {
        const float kq = sm.scal[1];
        const float o0 = a.scale * (dq[0] + u[0] * kq), o1 = a.scale * (dq[1] + u[1] * kq);
        *reinterpret_cast<uint32_t *>(a.out + row * kV + col) =
            (uint32_t)f32_to_bf16_bits(o0) | ((uint32_t)f32_to_bf16_bits(o1) << 16);
    }
    // ---- S' = D + k u^T ----------------------------------------------------
    if (a.ht) {
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            const int c = kRows * rg + i;
            const float kc = sm.kh[c];
            const float s0 = D[i][0] + kc * u[0], s1 = D[i][1] + kc * u[1];
            const int64_t idx = sbase + (int64_t)c * kV;
            if (a.ht_bf16) {
                state_store<kNT>(reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(a.ht) + idx),
                                 (uint32_t)f32_to_bf16_bits(s0) | ((uint32_t)f32_to_bf16_bits(s1) << 16));
            } else {
                state_store<kNT>(reinterpret_cast<f2 *>(reinterpret_cast<float *>(a.ht) + idx), (f2{s0, s1}));
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) void kda_decode_kernel(DecodeArgs a) { decode_body<false, 1>(a); }
__global__ __launch_bounds__(kThreads) void kda_decode_stream_kernel(DecodeArgs a) { decode_body<true, 1>(a); }
__global__ __launch_bounds__(kThreads) void kda_decode_split2_kernel(DecodeArgs a) { decode_body<false, 2>(a); }
__global__ __launch_bounds__(kThreads) void kda_decode_split4_kernel(DecodeArgs a) { decode_body<false, 4>(a); }

}  // namespace

// (sequence, head) units per launch of the one-slice kernels: at most 2^22
// workgroups of 256 threads, i.e. 2^30 work-items (a dispatch's grid is
// counted in 32-bit work-items per dimension).  The sliced kernels are only
// used for at most 1024 workgroups.
constexpr int64_t kMaxUnitsPerLaunch = int64_t(1) << 22;

hipError_t kda_launch_decode(const DecodeArgs &a, hipStream_t s) {
    const int64_t units = a.N * a.H;
    if (units <= 0) return hipSuccess;
    DecodeArgs b = a;
    b.unit_base = 0;
    const int64_t elt = (a.h0 && !a.h0_bf16) || (a.ht && !a.ht_bf16) ? 4 : 2;
    const bool stream = units * kK * kV * elt >= kStreamStateBytes;
    const bool forced = a.piece_cap > 0;
    const int64_t piece = launch_piece(kMaxUnitsPerLaunch, a.piece_cap);
    if (!stream && !forced && units * 4 <= kSplitWorkgroups) {
        hipLaunchKernelGGL(kda_decode_split4_kernel, dim3((unsigned)(units * 4)), dim3(kThreads), 0, s, b);
        return hipGetLastError();
    }
    if (!stream && !forced && units * 2 <= 2 * kSplitWorkgroups) {
        hipLaunchKernelGGL(kda_decode_split2_kernel, dim3((unsigned)(units * 2)), dim3(kThreads), 0, s, b);
        return hipGetLastError();
    }
    for (int64_t u0 = 0; u0 < units; u0 += piece) {
        const int64_t nu = units - u0 < piece ? units - u0 : piece;
        b.unit_base = u0;
        if (stream)
            hipLaunchKernelGGL(kda_decode_stream_kernel, dim3((unsigned)nu), dim3(kThreads), 0, s, b);
        else
            hipLaunchKernelGGL(kda_decode_kernel, dim3((unsigned)nu), dim3(kThreads), 0, s, b);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}
