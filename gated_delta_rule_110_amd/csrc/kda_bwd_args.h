// kda_bwd_args.h -- internal definitions of the backward pass (kda_bwd.hip and
// its launch in kda_api.hip), kept apart from kda_common.h so that the forward
// kernels do not depend on them.  Not part of the public ABI.
#pragma once
#include "kda_common.h"

namespace kda {

// The backward pass (kda_bwd.hip).  Per (chunk slot, head) unit ws = slot * H + h
// the workspace holds, besides the forward's fragment intermediates:
//   hs, dhs [ws][K][V] fp32   state entering the chunk / gradient of the state leaving it
//   dUt     [ws][64][V] fp32  gradient of the chunk's pseudo-values Ut = U - W S
//   G [ws][64][K] fp32          cumulative log-decay within the chunk
//   rq, rk, bb [ws][64] fp32    reciprocal norms of q and k (the normalised rows are
//                               recomputed from q and k where needed), b = sigmoid(beta)
//   Mk, Tm [ws][64][64] fp32    decayed key Gram (strictly lower, without b) and T = (I + Diag(b) Mk)^-1
//   part [ws][K + 1] fp32       this chunk's share of ddt_bias (K) and of dA_log (1)
//   co [ws][57856 B]            the reverse chain's fp16 operands (layout in kda_bwd.hip)
// Rows past the end of a ragged chunk are zero in rq, rk, bb and keep G constant.
constexpr int64_t kBwdChainOperandBytes = 57856;  // per (chunk, head): the reverse chain's fp16 operands

struct BwdArgs {
    const uint16_t *q, *k, *v, *g, *beta;   // bf16 inputs
    const float *A_log, *dt_bias;
    float lower_bound, scale;
    const uint16_t *dout;                   // [B,T,H,V] bf16, gradient of out
    const void *dht;                        // [N,H,K,V] gradient of the final state, or nullptr
    int dht_bf16;
    const int64_t *cu;
    const int32_t *chunk_off, *seq_order;
    int64_t T, H, N, nc_fixed, slots;
    const _Float16 *Wf, *Qf, *Kf, *Af;      // the forward's intermediates
    const float *gn;
    float *hs, *dhs, *dUt, *G, *rq, *rk, *bb, *Mk, *Tm, *part;
    unsigned char *co;                      // [ws][57856 B] the reverse chain's fp16 operands
    float *dq, *dk, *dv, *dg, *dbeta;       // [B,T,H,K] / [B,T,H,V] / [B,T,H] fp32
    float *dh0;                             // [N,H,K,V] fp32 or nullptr
    float *dA_log, *ddt_bias;               // [H] / [H,K] fp32
    // Map mode of the reverse chain (chain_map != 0): it stores neither dhs nor
    // dUt, only the gradient entering every sequence (dh0): with no gradient
    // of the final state (dht null) that is the offset of a segment's map.
    int chain_map;
    int64_t unit_base, chain_base;          // first unit / chain of a launch; set by the launchers
    int64_t piece_cap;                      // kda_desc_t::launch_piece (0: launch size by the default rule)
};

}  // namespace kda

// The backward's own kernels (kda_bwd.hip), in this order: per-chunk
// preparation, the reverse state chain (over BwdArgs' sequences, which may be
// the segments of split chains), then the per-chunk gradient and the sum of the
// shared parameters' partial gradients.
hipError_t kda_launch_bwd_prep(const kda::BwdArgs &a, hipStream_t s);
hipError_t kda_launch_bwd_chain(const kda::BwdArgs &a, hipStream_t s);
hipError_t kda_launch_bwd_grad(const kda::BwdArgs &a, hipStream_t s);
