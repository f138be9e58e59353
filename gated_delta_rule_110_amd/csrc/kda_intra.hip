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
// decay).  The state-chain kernel consumes W, U, Kbar, Qg, A_qk and exp(G_n),
// which this kernel writes in MFMA fragment order (see kda_common.h).
//
// Wave w owns rows 16 w .. 16 w + 15; lane (r, g) holds row 16 w + r and the
// channels 32 kk + 8 g + e (kk = 0..3, e = 0..7), which is the A/B operand
// layout of a 16x16x32 MFMA over channels.
//
// Decay factors exp(G_i - G_j) are never formed as exp(G_i) * exp(-G_j) over a
// whole chunk (that overflows): within each 16-row block r..r+15 the kernel
// keeps P_i = exp(G_i - G_{r-1}) (a product of at most 16 factors >= exp(-5),
// so >= exp(-80) > FLT_MIN), and off-diagonal 16x16 blocks use the row
// block's start as the reference so that both MFMA factors are <= 1 (fp16).
// The diagonal blocks, whose factors span up to exp(+-80), use bf16 hi + lo
// splits (three bf16 MFMAs).  That is what the lower bound of -5 on the
// log-decay buys.
//
// Layout changes between the token-major rows a lane holds and the
// channel-major or 4-token fragments the products need are done on the matrix
// cores: an MFMA against a 0/1 selection matrix moves fp16 values exactly.
//
// The triangular inverse: the 16x16 diagonal blocks by forward substitution
// in fp32, then the off-diagonal blocks column block by column block, each
// wave keeping its column of T in MFMA registers (split-fp16 products), so no
// barrier separates the block rows.
#include "kda_intra_body.h"

using namespace kda;

namespace {

template <bool kStream>
__global__ __launch_bounds__(intra::kThreads, 2) void kda_intra_kernel(IntraArgs a) {
    __shared__ intra::IntraSmem sm;

    // Heads fastest where the grid allows (gridDim.y <= 65535 chunk slots): the
    // workgroups in flight together then cover whole token rows, and the chain
    // kernel that runs next reads the intermediates measurably faster.
    const int64_t slot = a.slot_base + (a.heads_fast ? blockIdx.y : blockIdx.x);
    const int64_t h = a.heads_fast ? blockIdx.x : blockIdx.y;
    intra::intra_chunk<kStream>(a, slot, h, sm, (int)threadIdx.x, [] { lds_barrier(); });
}

// Intermediates of at least 128 MiB (this many chunk-heads) are written with
// the non-temporal hint on their 16-byte stores (W, Q_gamma, A_qk).  From this
// size on, the kernel's inputs and intermediates together outgrow the 256 MB
// Infinity Cache, so the intermediates cannot wait there for the chain kernel
// anyway.  Written past it, they leave no dirty lines in the cache for the
// chain's reads to evict (the likely reason), and the chain runs 2-5% faster
// (one 8K-token sequence at H = 32: 135 -> 129 us).  Below it they are read
// back from the cache, and the hint would cost 5-13% of the forward.  (On the
// 8-byte K-bar stores, whose halves come from two waves, the hint slowed this
// kernel by 2%; on the U stores it changed nothing.)
constexpr int64_t kInterBytesPerChunkHead =
    2 * (kWfElems + kQfElems + kKfElems + kAfElems + kUfElems) + 4 * kGnElems;
constexpr int64_t kStreamChunkHeads = ((int64_t(128) << 20) + kInterBytesPerChunkHead - 1) / kInterBytesPerChunkHead;

// Above 65535 chunk slots the grid is (slots, H), launched in pieces of at
// most 2^22 slots so that a launch stays within 2^30 work-items in x (a
// dispatch's grid is counted in 32-bit work-items per dimension).
constexpr int64_t kMaxSlotsPerLaunch = int64_t(1) << 22;

template <bool kStream>
hipError_t launch_intra(const IntraArgs &a, int64_t slots, hipStream_t s) {
    IntraArgs b = a;
    const bool forced = a.piece_cap > 0;
    const int64_t piece = launch_piece(kMaxSlotsPerLaunch, a.piece_cap);
    b.heads_fast = slots <= 65535 && a.H <= 65535 && !forced;
    if (b.heads_fast) {
        b.slot_base = 0;
        hipLaunchKernelGGL(kda_intra_kernel<kStream>, dim3((unsigned)a.H, (unsigned)slots), dim3(intra::kThreads), 0, s, b);
        return hipGetLastError();
    }
    for (int64_t s0 = 0; s0 < slots; s0 += piece) {
        const int64_t ns = slots - s0 < piece ? slots - s0 : piece;
        b.slot_base = s0;
        hipLaunchKernelGGL(kda_intra_kernel<kStream>, dim3((unsigned)ns, (unsigned)a.H), dim3(intra::kThreads), 0, s, b);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t kda_launch_intra(const IntraArgs &a, int64_t slots, hipStream_t s) {
    if (slots <= 0) return hipSuccess;
    if (slots * a.H >= kStreamChunkHeads) return launch_intra<true>(a, slots, s);
    return launch_intra<false>(a, slots, s);
}
