// kda_api.hip -- the C ABI of libkda: validation, workspace carving, launches.
//
// Argument list, dtypes and the K = V = 128 restriction follow the forward
// call described on "Debajo del capó: CUTLASS en Hopper" (7minutos.es); the
// contiguity / same-device requirements follow "性能与注意事项"
// (zuobiaodaohang.com FlashKDA page).
#include <math.h>
#include "kda_common.h"
#include "kda.h"

using namespace kda;

namespace {

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Fills geometry; returns KDA_OK or the shape error.
kda_status_t make_geometry(const kda_desc_t *d, bool varlen, Geometry &g) {
    if (d->B < 1 || d->H < 1 || d->T < 0) return KDA_ERR_SHAPE;
    if (d->K != kK || d->V != kV) return KDA_ERR_UNSUPPORTED;
    if (d->H > 65535) return KDA_ERR_SHAPE;  // grid y dimension
    g.B = d->B; g.T = d->T; g.H = d->H; g.varlen = varlen;
    const int64_t nc = (d->T + kChunk - 1) / kChunk;
    if (varlen) {
        if (d->B != 1 || d->num_seqs < 1) return KDA_ERR_SHAPE;
        g.N = d->num_seqs;
        g.nc_fixed = 0;
        g.slots = nc + g.N;
    } else {
        if (d->num_seqs != d->B) return KDA_ERR_SHAPE;
        g.N = d->B;
        g.nc_fixed = nc;
        g.slots = g.N * nc;
    }
    if (g.slots > 0x7fffffffLL || g.N > 0x7fffffffLL) return KDA_ERR_SHAPE;
    return KDA_OK;
}

WorkspaceLayout make_layout(const Geometry &g) {
    WorkspaceLayout L{};
    const size_t per = (size_t)g.slots * (size_t)g.H;
    size_t o = 0;
    L.off_chunk_off = o; o = align_up(o + (g.varlen ? sizeof(int32_t) * (size_t)(g.N + 1) : 0), 256);
    L.off_Wf = o; o = align_up(o + per * kWfElems * 2, 256);
    L.off_Qf = o; o = align_up(o + per * kQfElems * 2, 256);
    L.off_Kf = o; o = align_up(o + per * kKfElems * 2, 256);
    L.off_Af = o; o = align_up(o + per * kAfElems * 2, 256);
    L.off_Uf = o; o = align_up(o + per * kUfElems * 2, 256);
    L.off_gn = o;  o = align_up(o + per * kGnElems * 4, 256);
    L.total = o;
    return L;
}

}  // namespace

extern "C" size_t kda_fwd_workspace_size(const kda_desc_t *desc) {
    if (!desc) return 0;
    // The descriptor does not say whether cu_seqlens will be passed, so with
    // B == 1 the larger of the packed and unpacked layouts is returned.
    Geometry g;
    size_t need = 0;
    bool ok = false;
    if (make_geometry(desc, false, g) == KDA_OK) { need = make_layout(g).total; ok = true; }
    if (desc->B == 1 && make_geometry(desc, true, g) == KDA_OK) {
        const size_t p = make_layout(g).total;
        need = p > need ? p : need;
        ok = true;
    }
    return ok ? need : 0;
}

extern "C" const char *kda_status_string(kda_status_t s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL: return "a required pointer is NULL";
        case KDA_ERR_SHAPE: return "invalid shape (B, H >= 1, T >= 0; num_seqs == B, or B == 1 with cu_seqlens)";
        case KDA_ERR_UNSUPPORTED: return "unsupported head dimension (K and V must be 128)";
        case KDA_ERR_PARAM: return "invalid parameter (lower_bound must be finite and in [-5, 0]; scale finite)";
        case KDA_ERR_DTYPE: return "state dtype must be KDA_BF16 or KDA_FP32";
        case KDA_ERR_ALIGN: return "misaligned pointer (tensors 16 bytes, workspace 256 bytes)";
        case KDA_ERR_WORKSPACE: return "workspace smaller than kda_fwd_workspace_size()";
        case KDA_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

extern "C" kda_status_t kda_fwd(const void *q, const void *k, const void *v, const void *g,
                                const void *beta, float scale, const float *A_log,
                                const float *dt_bias, float lower_bound,
                                const void *initial_state, void *final_state,
                                const int64_t *cu_seqlens, void *out,
                                const kda_desc_t *desc, hipStream_t stream) {
    if (!desc || !A_log || !dt_bias) return KDA_ERR_NULL;
    Geometry geo;
    kda_status_t st = make_geometry(desc, cu_seqlens != nullptr, geo);
    if (st != KDA_OK) return st;
    // token tensors hold B*T rows; with no tokens they may be empty (NULL)
    if (geo.T > 0 && (!q || !k || !v || !g || !beta || !out)) return KDA_ERR_NULL;
    if (!(lower_bound >= -5.0f && lower_bound <= 0.0f)) return KDA_ERR_PARAM;  // also rejects NaN
    if (!isfinite(scale)) return KDA_ERR_PARAM;
    if (initial_state && desc->initial_state_dtype != KDA_BF16 && desc->initial_state_dtype != KDA_FP32)
        return KDA_ERR_DTYPE;
    if (final_state && desc->final_state_dtype != KDA_BF16 && desc->final_state_dtype != KDA_FP32)
        return KDA_ERR_DTYPE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(g, 16) || !aligned(out, 16) ||
        !aligned(dt_bias, 16) || !aligned(beta, 2) || !aligned(A_log, 4) ||
        (cu_seqlens && !aligned(cu_seqlens, 8)) ||
        (initial_state && !aligned(initial_state, 4)) || (final_state && !aligned(final_state, 4)))
        return KDA_ERR_ALIGN;
    const WorkspaceLayout lay = make_layout(geo);
    char *ws = static_cast<char *>(desc->workspace);
    bool owned = false;
    if (ws) {
        if (!aligned(ws, 256)) return KDA_ERR_ALIGN;
        if (desc->workspace_bytes < lay.total) return KDA_ERR_WORKSPACE;
    } else if (lay.total > 0) {
        void *p = nullptr;
        if (hipMallocAsync(&p, lay.total, stream) != hipSuccess) return KDA_ERR_HIP;
        ws = static_cast<char *>(p);
        owned = true;
    }

    hipEvent_t *ev = desc->phase_events;
    int32_t *chunk_off = geo.varlen ? reinterpret_cast<int32_t *>(ws + lay.off_chunk_off) : nullptr;
    hipError_t err = hipSuccess;
    if (ev) err = hipEventRecord(ev[0], stream);
    if (err == hipSuccess && geo.varlen) err = kda_launch_chunk_table(cu_seqlens, geo.N, chunk_off, stream);
    if (ev && err == hipSuccess) err = hipEventRecord(ev[1], stream);

    IntraArgs ia{};
    ia.q = static_cast<const uint16_t *>(q); ia.k = static_cast<const uint16_t *>(k);
    ia.v = static_cast<const uint16_t *>(v); ia.g = static_cast<const uint16_t *>(g);
    ia.beta = static_cast<const uint16_t *>(beta);
    ia.A_log = A_log; ia.dt_bias = dt_bias; ia.lower_bound = lower_bound;
    ia.cu = cu_seqlens; ia.chunk_off = chunk_off;
    ia.T = geo.T; ia.H = geo.H; ia.N = geo.N; ia.nc_fixed = geo.nc_fixed;
    ia.Wf = reinterpret_cast<_Float16 *>(ws + lay.off_Wf);
    ia.Qf = reinterpret_cast<_Float16 *>(ws + lay.off_Qf);
    ia.Kf = reinterpret_cast<_Float16 *>(ws + lay.off_Kf);
    ia.Af = reinterpret_cast<_Float16 *>(ws + lay.off_Af);
    ia.Uf = reinterpret_cast<_Float16 *>(ws + lay.off_Uf);
    ia.gn = reinterpret_cast<float *>(ws + lay.off_gn);
    if (err == hipSuccess && geo.T > 0) err = kda_launch_intra(ia, geo.slots, stream);
    if (ev && err == hipSuccess) err = hipEventRecord(ev[2], stream);

    ChainArgs ca{};
    ca.Wf = ia.Wf; ca.Qf = ia.Qf; ca.Kf = ia.Kf; ca.Af = ia.Af; ca.Uf = ia.Uf; ca.gn = ia.gn;
    ca.cu = cu_seqlens; ca.chunk_off = chunk_off;
    ca.T = geo.T; ca.H = geo.H; ca.N = geo.N; ca.nc_fixed = geo.nc_fixed;
    ca.scale = scale;
    ca.h0 = initial_state; ca.ht = final_state;
    ca.h0_bf16 = desc->initial_state_dtype == KDA_BF16;
    ca.ht_bf16 = desc->final_state_dtype == KDA_BF16;
    ca.out = static_cast<uint16_t *>(out);
    if (err == hipSuccess) err = kda_launch_chain(ca, stream);
    if (ev && err == hipSuccess) err = hipEventRecord(ev[3], stream);

    if (owned) {
        hipError_t e2 = hipFreeAsync(ws, stream);
        if (err == hipSuccess) err = e2;
    }
    return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

extern "C" kda_status_t kda_decode(const void *q, const void *k, const void *v, const void *g,
                                   const void *beta, float scale, const float *A_log,
                                   const float *dt_bias, float lower_bound,
                                   const void *initial_state, void *final_state, void *out,
                                   const kda_desc_t *desc, hipStream_t stream) {
    if (!desc || !A_log || !dt_bias) return KDA_ERR_NULL;
    if (desc->B < 1 || desc->H < 1 || desc->T != 1 || desc->num_seqs != desc->B) return KDA_ERR_SHAPE;
    if (desc->K != kK || desc->V != kV) return KDA_ERR_UNSUPPORTED;
    if (desc->B * desc->H > 0xffffffffLL) return KDA_ERR_SHAPE;
    if (!q || !k || !v || !g || !beta || !out) return KDA_ERR_NULL;
    if (!(lower_bound >= -5.0f && lower_bound <= 0.0f)) return KDA_ERR_PARAM;
    if (!isfinite(scale)) return KDA_ERR_PARAM;
    if (initial_state && desc->initial_state_dtype != KDA_BF16 && desc->initial_state_dtype != KDA_FP32)
        return KDA_ERR_DTYPE;
    if (final_state && desc->final_state_dtype != KDA_BF16 && desc->final_state_dtype != KDA_FP32)
        return KDA_ERR_DTYPE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(g, 16) || !aligned(out, 16) ||
        !aligned(dt_bias, 16) || !aligned(beta, 2) || !aligned(A_log, 4) ||
        (initial_state && !aligned(initial_state, 8)) || (final_state && !aligned(final_state, 8)))
        return KDA_ERR_ALIGN;
    DecodeArgs da{};
    da.q = static_cast<const uint16_t *>(q); da.k = static_cast<const uint16_t *>(k);
    da.v = static_cast<const uint16_t *>(v); da.g = static_cast<const uint16_t *>(g);
    da.beta = static_cast<const uint16_t *>(beta);
    da.A_log = A_log; da.dt_bias = dt_bias; da.lower_bound = lower_bound; da.scale = scale;
    da.N = desc->B; da.H = desc->H;
    da.h0 = initial_state; da.ht = final_state;
    da.h0_bf16 = desc->initial_state_dtype == KDA_BF16;
    da.ht_bf16 = desc->final_state_dtype == KDA_BF16;
    da.out = static_cast<uint16_t *>(out);
    return kda_launch_decode(da, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}
