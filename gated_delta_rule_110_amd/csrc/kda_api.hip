// kda_api.hip -- the C ABI of libkda: validation, workspace carving, launches.
//
// Argument list, dtypes and the K = V = 128 restriction follow the forward
// call described on "Debajo del capó: CUTLASS en Hopper" (7minutos.es); the
// contiguity / same-device requirements follow "性能与注意事项"
// (zuobiaodaohang.com FlashKDA page).
#include <math.h>
#include <stdlib.h>
#include <mutex>
#include <vector>
#include "kda_bwd_args.h"
#include "kda.h"

using namespace kda;

namespace {

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// How many segments each sequence's state chain is cut into (kda.h,
// kda_desc_t::chain_segments).  Automatic splitting gives every (segment,
// head) 8 workgroups and takes the larger of two counts: one round of
// workgroups over the 256 CUs with at least 32 chunks per segment, or two
// rounds with at least 64 chunks per segment.  Two rounds measured faster
// wherever their segments stay that long (one 128K-token sequence: H = 4
// 722 -> 682 us, H = 8 1351 -> 1237 us, H = 12 2607 -> 1886 us unsplit before,
// H = 16 2801 -> 2389 us unsplit before), one round where they would not
// (H = 1: 32 segments 252 us, 64 segments 318 us).  A split runs every chunk
// twice (the map pass and the chain pass), so it pays from 3 segments on
// (H = 20: 3 segments 3118 us against 3176 unsplit; H = 24 and 32: 2 segments
// 22% slower than none).
constexpr int64_t kCUs = 256;
constexpr int64_t kChainWorkgroups = 8;
constexpr int64_t kMinSegmentChunks = 32;
constexpr int64_t kMinAutoSegments = 3;

kda_status_t choose_segments(const kda_desc_t *d, Geometry &g) {
    g.segs = 1;
    g.segc = g.nc_fixed;
    const int64_t req = d->chain_segments;
    if (req < 0) return KDA_ERR_PARAM;
    if (g.varlen) return req >= 2 ? KDA_ERR_UNSUPPORTED : KDA_OK;
    const int64_t nc = g.nc_fixed;
    int64_t want = req;
    if (req == 0) {
        const int64_t bh = g.B * g.H;
        int64_t one = kCUs / kChainWorkgroups / bh;
        if (one > nc / kMinSegmentChunks) one = nc / kMinSegmentChunks;
        int64_t two = 2 * kCUs / kChainWorkgroups / bh;
        if (two > nc / (2 * kMinSegmentChunks)) two = nc / (2 * kMinSegmentChunks);
        want = one > two ? one : two;
        if (want < kMinAutoSegments) want = 1;
    }
    if (want > nc) want = nc;
    if (want < 2) return KDA_OK;
    g.segc = (nc + want - 1) / want;
    g.segs = (nc + g.segc - 1) / g.segc;  // >= 2: segc < nc when 2 <= want <= nc
    return KDA_OK;
}

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
    if (d->pipeline < 0 || d->pipeline > 1) return KDA_ERR_PARAM;
    if (d->save_states < 0 || d->save_states > 1) return KDA_ERR_PARAM;
    const kda_status_t st = choose_segments(d, g);
    g.fused = st == KDA_OK && g.segs == 1 && d->pipeline == 1 && d->save_states == 0 &&
              kda_fused_applies(g.N, g.H, g.varlen);
    return st;
}

WorkspaceLayout make_layout(const Geometry &g) {
    WorkspaceLayout L{};
    const size_t per = (size_t)g.slots * (size_t)g.H;
    size_t o = 0;
    L.off_chunk_off = o; o = align_up(o + (g.varlen ? sizeof(int32_t) * (size_t)(g.N + 1) : 0), 256);
    L.off_seq_order = o; o = align_up(o + (g.varlen ? sizeof(int32_t) * (size_t)g.N : 0), 256);
    L.off_Wf = o; o = align_up(o + per * kWfElems * 2, 256);
    L.off_Qf = o; o = align_up(o + per * kQfElems * 2, 256);
    L.off_Kf = o; o = align_up(o + per * kKfElems * 2, 256);
    L.off_Af = o; o = align_up(o + per * kAfElems * 2, 256);
    L.off_Uf = o; o = align_up(o + per * kUfElems * 2, 256);
    L.off_gn = o;  o = align_up(o + per * kGnElems * 4, 256);
    if (g.segs > 1) {
        const size_t ns = (size_t)(g.B * g.segs);
        const size_t maps = ns * (size_t)g.H * (size_t)(kK * kV) * 4;
        L.off_seg_cu = o;  o = align_up(o + (ns + 1) * sizeof(int64_t), 256);
        L.off_seg_off = o; o = align_up(o + (ns + 1) * sizeof(int32_t), 256);
        L.off_mapM = o;    o = align_up(o + maps, 256);
        L.off_mapN = o;    o = align_up(o + maps, 256);
        L.off_sin = o;     o = align_up(o + maps, 256);
    }
    if (g.fused) {
        L.off_flags = o; o = align_up(o + per * sizeof(int32_t), 256);
        L.off_error = o; o = align_up(o + sizeof(int32_t), 256);
        L.off_counters = o; o = align_up(o + 8 * sizeof(unsigned long long), 256);
    }
    L.total = o;
    return L;
}

// Bytes of the fp32 states entering every chunk slot that kda_fwd stores past
// the end of its layout with kda_desc_t::save_states = 1.
size_t saved_states_bytes(const Geometry &g) {
    return align_up((size_t)g.slots * (size_t)g.H * (size_t)(kK * kV) * 4, 256);
}

// kda_fwd's workspace: its layout, and the saved states after it.
size_t fwd_workspace_bytes(const kda_desc_t *d, const Geometry &g) {
    return make_layout(g).total + (d->save_states == 1 ? saved_states_bytes(g) : 0);
}

// With KDA_VALIDATE=1 in the environment, kda_fwd reads cu_seqlens back to the
// host (synchronising `stream`) and refuses contents that would send the
// kernels outside the token tensors.  Off by default: it costs a device
// round trip and cannot be captured in a graph.
bool validate_requested() {
    const char *e = getenv("KDA_VALIDATE");
    return e && e[0] == '1' && e[1] == 0;
}

kda_status_t validate_cu_seqlens(const int64_t *cu, int64_t N, int64_t T, hipStream_t stream) {
    std::vector<int64_t> h((size_t)N + 1);
    if (hipMemcpyAsync(h.data(), cu, sizeof(int64_t) * (size_t)(N + 1), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return KDA_ERR_HIP;
    if (h[0] != 0 || h[(size_t)N] != T) return KDA_ERR_SHAPE;
    for (int64_t n = 0; n < N; ++n)
        if (h[(size_t)n + 1] < h[(size_t)n]) return KDA_ERR_SHAPE;
    return KDA_OK;
}

}  // namespace

extern "C" size_t kda_fwd_workspace_size(const kda_desc_t *desc) {
    if (!desc) return 0;
    // The descriptor does not say whether cu_seqlens will be passed, so with
    // B == 1 the larger of the packed and unpacked layouts is returned.
    Geometry g;
    size_t need = 0;
    bool ok = false;
    if (make_geometry(desc, false, g) == KDA_OK) { need = fwd_workspace_bytes(desc, g); ok = true; }
    if (desc->B == 1 && make_geometry(desc, true, g) == KDA_OK) {
        const size_t p = fwd_workspace_bytes(desc, g);
        need = p > need ? p : need;
        ok = true;
    }
    return ok ? need : 0;
}

extern "C" int64_t kda_fwd_chain_segments(const kda_desc_t *desc) {
    if (!desc) return -1;
    Geometry g;
    if (make_geometry(desc, false, g) != KDA_OK) return -1;
    return g.segs;
}

extern "C" int kda_fwd_pipelined(const kda_desc_t *desc) {
    if (!desc) return -1;
    Geometry g;
    if (make_geometry(desc, false, g) != KDA_OK) return -1;
    return g.fused ? 1 : 0;
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
        case KDA_ERR_SCRATCH: return "workspace need exceeds the static scratch of kda_fwd_noalloc (kda_fwd_noalloc_max_workspace() bytes)";
    }
    return "unknown status";
}

// Static scratch of kda_fwd_noalloc: the workspace of its calls, in the code
// object's own device memory, so that the call needs no allocation.  Host code
// must never pass `scratch` itself to a kernel or a copy: in host code the name
// stands for a host-side shadow, not for the device array.  Its device address
// is looked up once per device with hipGetSymbolAddress (scratch_on_device) and
// only that address is used.
constexpr size_t kScratchBytes = size_t(128) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

void *scratch_on_device(int dev);

// The split chains' view of a batch: segment s of batch row b is packed
// sequence b * segs + s (its token and chunk ranges from the segment table).
struct SegmentView {
    int64_t *cu;
    int32_t *off;
    float *mapM, *mapN, *sin;
};

SegmentView segment_view(const WorkspaceLayout &lay, char *ws) {
    SegmentView v;
    v.cu = reinterpret_cast<int64_t *>(ws + lay.off_seg_cu);
    v.off = reinterpret_cast<int32_t *>(ws + lay.off_seg_off);
    v.mapM = reinterpret_cast<float *>(ws + lay.off_mapM);
    v.mapN = reinterpret_cast<float *>(ws + lay.off_mapN);
    v.sin = reinterpret_cast<float *>(ws + lay.off_sin);
    return v;
}

// The forward's state chains: one launch, or with split chains the segment
// table, the map of every segment, the scan over the segments (the entering
// states and ca.ht) and the chain from every segment's entering state.  With
// ca.hs set the chain also stores the state entering every chunk.
hipError_t launch_chains(const ChainArgs &ca, const Geometry &geo, const WorkspaceLayout &lay, char *ws,
                         hipStream_t stream) {
    if (geo.segs <= 1) return kda_launch_chain(ca, stream);
    const SegmentView sv = segment_view(lay, ws);
    ChainArgs seg = ca;
    seg.cu = sv.cu; seg.chunk_off = sv.off; seg.seq_order = nullptr;
    seg.N = geo.B * geo.segs; seg.nc_fixed = 0;
    hipError_t err = kda_launch_seg_table(geo.B, geo.T, geo.segs, geo.segc, sv.cu, sv.off, stream);
    ChainArgs maps = seg;  // 1. the map of every segment
    maps.h0 = nullptr; maps.ht = nullptr; maps.out = nullptr; maps.hs = nullptr;
    maps.map_mode = 1; maps.mapM = sv.mapM; maps.mapN = sv.mapN;
    if (err == hipSuccess) err = kda_launch_chain(maps, stream);
    ScanArgs sa{};     // 2. entering states and the final state
    sa.mapM = sv.mapM; sa.mapN = sv.mapN; sa.sin = sv.sin;
    sa.h0 = ca.h0; sa.ht = ca.ht;
    sa.h0_bf16 = ca.h0_bf16; sa.ht_bf16 = ca.ht_bf16;
    sa.B = geo.B; sa.H = geo.H; sa.segs = geo.segs;
    if (err == hipSuccess) err = kda_launch_seg_scan(sa, stream);
    seg.h0 = sv.sin; seg.h0_bf16 = 0; seg.ht = nullptr;  // 3. outputs
    if (err == hipSuccess) err = kda_launch_chain(seg, stream);
    return err;
}

// The gradient's reverse state chains.  With split chains: the reverse chain of
// every segment from a zero gradient (the offsets of the segments' reverse maps,
// into mapN, whose forward contents the forward scan has consumed), the
// reverse scan with the transposed forward maps (the gradient leaving every
// segment, into sin, and the gradient of the initial state), and the reverse
// chain of every segment from the gradient leaving it.
// The segment table and the forward's segment maps come from `fws`, the
// workspace the forward's chains ran in (the call's own, or the kept forward
// workspace when that call's states are read).
hipError_t launch_bwd_chains(const BwdArgs &ba, const Geometry &geo, const WorkspaceLayout &lay, char *ws,
                             char *fws, hipStream_t stream) {
    if (geo.segs <= 1) return kda_launch_bwd_chain(ba, stream);
    SegmentView sv = segment_view(lay, ws);
    const SegmentView fv = segment_view(lay, fws);
    sv.cu = fv.cu; sv.off = fv.off; sv.mapM = fv.mapM;
    BwdArgs seg = ba;
    seg.cu = sv.cu; seg.chunk_off = sv.off; seg.seq_order = nullptr;
    seg.N = geo.B * geo.segs; seg.nc_fixed = 0;
    BwdArgs maps = seg;  // 1. offsets
    maps.chain_map = 1; maps.dht = nullptr; maps.dh0 = sv.mapN;
    hipError_t err = kda_launch_bwd_chain(maps, stream);
    ScanArgs sa{};       // 2. the gradient leaving every segment; the initial state's
    sa.mapM = sv.mapM; sa.mapN = sv.mapN; sa.sin = sv.sin;
    sa.h0 = ba.dht; sa.h0_bf16 = ba.dht_bf16;
    sa.ht = ba.dh0; sa.ht_bf16 = 0;
    sa.reverse = 1;
    sa.B = geo.B; sa.H = geo.H; sa.segs = geo.segs;
    if (err == hipSuccess) err = kda_launch_seg_scan(sa, stream);
    seg.dht = sv.sin; seg.dht_bf16 = 0; seg.dh0 = nullptr;  // 3. per-chunk gradients
    if (err == hipSuccess) err = kda_launch_bwd_chain(seg, stream);
    return err;
}

// The forward pass behind kda_fwd and kda_fwd_noalloc.  With `noalloc` the
// call runs in the library's static scratch (the descriptor's workspace is
// ignored) and allocates nothing, on the device or the host; otherwise it runs
// in the caller's workspace or one taken with hipMallocAsync.
kda_status_t fwd_impl(const void *q, const void *k, const void *v, const void *g, const void *beta,
                      float scale, const float *A_log, const float *dt_bias, float lower_bound,
                      const void *initial_state, void *final_state, const int64_t *cu_seqlens, void *out,
                      const kda_desc_t *desc, bool noalloc, hipStream_t stream) {
    if (!desc || !A_log || !dt_bias) return KDA_ERR_NULL;
    Geometry geo;
    kda_status_t st = make_geometry(desc, cu_seqlens != nullptr, geo);
    if (st != KDA_OK) return st;
    if (desc->launch_piece < 0) return KDA_ERR_PARAM;
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
    if (cu_seqlens && !noalloc && validate_requested()) {
        st = validate_cu_seqlens(cu_seqlens, geo.N, geo.T, stream);
        if (st != KDA_OK) return st;
    }
    if (noalloc && desc->save_states != 0) return KDA_ERR_PARAM;
    const WorkspaceLayout lay = make_layout(geo);
    const size_t need = fwd_workspace_bytes(desc, geo);
    char *ws = noalloc ? nullptr : static_cast<char *>(desc->workspace);
    bool owned = false;
    if (noalloc) {
        if (lay.total > kScratchBytes) return KDA_ERR_SCRATCH;
        int dev = -1;
        if (hipGetDevice(&dev) != hipSuccess) return KDA_ERR_HIP;
        ws = static_cast<char *>(scratch_on_device(dev));
        if (!ws) return KDA_ERR_HIP;
    } else if (ws) {
        if (!aligned(ws, 256)) return KDA_ERR_ALIGN;
        if (desc->workspace_bytes < need) return KDA_ERR_WORKSPACE;
    } else if (need > 0) {
        void *p = nullptr;
        if (hipMallocAsync(&p, need, stream) != hipSuccess) return KDA_ERR_HIP;
        ws = static_cast<char *>(p);
        owned = true;
    }

    hipEvent_t *ev = desc->phase_events;
    int32_t *chunk_off = geo.varlen ? reinterpret_cast<int32_t *>(ws + lay.off_chunk_off) : nullptr;
    int32_t *seq_order = geo.varlen ? reinterpret_cast<int32_t *>(ws + lay.off_seq_order) : nullptr;
    hipError_t err = hipSuccess;
    if (ev) err = hipEventRecord(ev[0], stream);
    if (err == hipSuccess && geo.varlen) err = kda_launch_chunk_table(cu_seqlens, geo.N, chunk_off, seq_order, stream);
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
    ia.piece_cap = desc->launch_piece;
    if (geo.fused) {
        // the pipelined forward: one grid for both sides (event 2 after it, event 3 right behind)
        ChainArgs ca{};
        ca.Wf = ia.Wf; ca.Qf = ia.Qf; ca.Kf = ia.Kf; ca.Af = ia.Af; ca.Uf = ia.Uf; ca.gn = ia.gn;
        ca.T = geo.T; ca.H = geo.H; ca.N = geo.N; ca.nc_fixed = geo.nc_fixed;
        ca.scale = scale;
        ca.h0 = initial_state; ca.ht = final_state;
        ca.h0_bf16 = desc->initial_state_dtype == KDA_BF16;
        ca.ht_bf16 = desc->final_state_dtype == KDA_BF16;
        ca.out = static_cast<uint16_t *>(out);
        if (err == hipSuccess && geo.T > 0)
            err = kda_launch_fused(ia, ca, reinterpret_cast<int32_t *>(ws + lay.off_flags),
                                   reinterpret_cast<int32_t *>(ws + lay.off_error),
                                   reinterpret_cast<unsigned long long *>(ws + lay.off_counters), geo.slots, stream);
        else if (err == hipSuccess) err = kda_launch_chain(ca, stream);  // T = 0: the states only
        if (ev && err == hipSuccess) err = hipEventRecord(ev[2], stream);
        if (ev && err == hipSuccess) err = hipEventRecord(ev[3], stream);
        if (owned) {
            hipError_t e2 = hipFreeAsync(ws, stream);
            if (err == hipSuccess) err = e2;
        }
        return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    if (err == hipSuccess && geo.T > 0) err = kda_launch_intra(ia, geo.slots, stream);
    if (ev && err == hipSuccess) err = hipEventRecord(ev[2], stream);

    ChainArgs ca{};
    ca.Wf = ia.Wf; ca.Qf = ia.Qf; ca.Kf = ia.Kf; ca.Af = ia.Af; ca.Uf = ia.Uf; ca.gn = ia.gn;
    ca.cu = cu_seqlens; ca.chunk_off = chunk_off; ca.seq_order = seq_order;
    ca.T = geo.T; ca.H = geo.H; ca.N = geo.N; ca.nc_fixed = geo.nc_fixed;
    ca.scale = scale;
    ca.h0 = initial_state; ca.ht = final_state;
    ca.h0_bf16 = desc->initial_state_dtype == KDA_BF16;
    ca.ht_bf16 = desc->final_state_dtype == KDA_BF16;
    ca.out = static_cast<uint16_t *>(out);
    // save_states: the chain also stores the state entering every chunk (past the layout's end)
    ca.hs = desc->save_states == 1 ? reinterpret_cast<float *>(ws + lay.total) : nullptr;
    ca.piece_cap = desc->launch_piece;
    if (err == hipSuccess) err = launch_chains(ca, geo, lay, ws, stream);
    if (ev && err == hipSuccess) err = hipEventRecord(ev[3], stream);

    if (owned) {
        hipError_t e2 = hipFreeAsync(ws, stream);
        if (err == hipSuccess) err = e2;
    }
    return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];

// The device address of this device's `scratch`, looked up on the first call
// with that device current; nullptr if the lookup fails.
void *scratch_on_device(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" kda_status_t kda_fwd(const void *q, const void *k, const void *v, const void *g,
                                const void *beta, float scale, const float *A_log,
                                const float *dt_bias, float lower_bound,
                                const void *initial_state, void *final_state,
                                const int64_t *cu_seqlens, void *out,
                                const kda_desc_t *desc, hipStream_t stream) {
    return fwd_impl(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, initial_state, final_state, cu_seqlens,
                    out, desc, false, stream);
}

extern "C" size_t kda_fwd_noalloc_max_workspace(void) { return kScratchBytes; }

extern "C" kda_status_t kda_fwd_noalloc(const void *q, const void *k, const void *v, const void *g,
                                        const void *beta, float scale, const float *A_log,
                                        const float *dt_bias, float lower_bound,
                                        const void *initial_state, void *final_state,
                                        const int64_t *cu_seqlens, void *out,
                                        const kda_desc_t *desc, hipStream_t stream) {
    return fwd_impl(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, initial_state, final_state, cu_seqlens,
                    out, desc, true, stream);
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
    if (desc->launch_piece < 0) return KDA_ERR_PARAM;
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
    da.piece_cap = desc->launch_piece;
    return kda_launch_decode(da, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// ---- backward -----------------------------------------------------------------

namespace {

struct BwdLayout {
    WorkspaceLayout fwd;  // the forward's intermediates (unsplit, two-kernel)
    size_t off_hs, off_dhs, off_dUt, off_G, off_rq, off_rk, off_bb, off_Mk, off_Tm, off_part,
        off_co;
    size_t total;
};

// Geometry of a backward call: the forward's (split chains by the same rule),
// never pipelined.
kda_status_t make_bwd_geometry(const kda_desc_t *d, bool varlen, Geometry &g) {
    if (d->save_states < 0 || d->save_states > 1) return KDA_ERR_PARAM;
    kda_desc_t e = *d;
    e.pipeline = 0;
    e.save_states = 0;
    return make_geometry(&e, varlen, g);
}

BwdLayout make_bwd_layout(const Geometry &g) {
    BwdLayout L{};
    L.fwd = make_layout(g);
    const size_t per = (size_t)g.slots * (size_t)g.H;
    size_t o = L.fwd.total;
    L.off_hs = o;   o = align_up(o + per * kK * kV * 4, 256);
    L.off_dhs = o;  o = align_up(o + per * kK * kV * 4, 256);
    L.off_dUt = o;  o = align_up(o + per * kChunk * kV * 4, 256);
    L.off_G = o;    o = align_up(o + per * kChunk * kK * 4, 256);
    L.off_rq = o;   o = align_up(o + per * kChunk * 4, 256);
    L.off_rk = o;   o = align_up(o + per * kChunk * 4, 256);
    L.off_bb = o;   o = align_up(o + per * kChunk * 4, 256);
    L.off_Mk = o;   o = align_up(o + per * kChunk * kChunk * 4, 256);
    L.off_Tm = o;   o = align_up(o + per * kChunk * kChunk * 4, 256);
    L.off_part = o; o = align_up(o + per * (kK + 1) * 4, 256);
    L.off_co = o;   o = align_up(o + per * kBwdChainOperandBytes, 256);
    L.total = o;
    return L;
}

}  // namespace

extern "C" size_t kda_bwd_workspace_size(const kda_desc_t *desc) {
    if (!desc) return 0;
    Geometry g;
    size_t need = 0;
    bool ok = false;
    if (make_bwd_geometry(desc, false, g) == KDA_OK) { need = make_bwd_layout(g).total; ok = true; }
    if (desc->B == 1 && make_bwd_geometry(desc, true, g) == KDA_OK) {
        const size_t p = make_bwd_layout(g).total;
        need = p > need ? p : need;
        ok = true;
    }
    return ok ? need : 0;
}

extern "C" kda_status_t kda_bwd(const void *q, const void *k, const void *v, const void *g,
                                const void *beta, float scale, const float *A_log,
                                const float *dt_bias, float lower_bound,
                                const void *initial_state, const int64_t *cu_seqlens,
                                const void *d_out, const void *d_final_state,
                                float *dq, float *dk, float *dv, float *dg, float *dbeta,
                                float *d_initial_state, float *dA_log, float *ddt_bias,
                                const kda_desc_t *desc, hipStream_t stream) {
    if (!desc || !A_log || !dt_bias || !dA_log || !ddt_bias) return KDA_ERR_NULL;
    Geometry geo;
    kda_status_t st = make_bwd_geometry(desc, cu_seqlens != nullptr, geo);
    if (st != KDA_OK) return st;
    if (desc->launch_piece < 0) return KDA_ERR_PARAM;
    if (geo.T > 0 && (!q || !k || !v || !g || !beta || !d_out || !dq || !dk || !dv || !dg || !dbeta))
        return KDA_ERR_NULL;
    if (!(lower_bound >= -5.0f && lower_bound <= 0.0f)) return KDA_ERR_PARAM;
    if (!isfinite(scale)) return KDA_ERR_PARAM;
    if (initial_state && desc->initial_state_dtype != KDA_BF16 && desc->initial_state_dtype != KDA_FP32)
        return KDA_ERR_DTYPE;
    if (d_final_state && desc->final_state_dtype != KDA_BF16 && desc->final_state_dtype != KDA_FP32)
        return KDA_ERR_DTYPE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(g, 16) || !aligned(d_out, 16) ||
        !aligned(dt_bias, 16) || !aligned(beta, 2) || !aligned(A_log, 4) ||
        !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(dg, 16) || !aligned(dbeta, 4) ||
        !aligned(dA_log, 4) || !aligned(ddt_bias, 4) ||
        (cu_seqlens && !aligned(cu_seqlens, 8)) || (initial_state && !aligned(initial_state, 4)) ||
        (d_final_state && !aligned(d_final_state, 4)) || (d_initial_state && !aligned(d_initial_state, 4)))
        return KDA_ERR_ALIGN;
    if (cu_seqlens && validate_requested()) {
        st = validate_cu_seqlens(cu_seqlens, geo.N, geo.T, stream);
        if (st != KDA_OK) return st;
    }
    const BwdLayout lay = make_bwd_layout(geo);
    // the forward's intermediates: recomputed into this call's workspace, or
    // those of the kda_fwd call that left them in desc->forward_workspace (the
    // intermediates sit at the same offsets in both layouts: make_layout puts
    // them before the parts that depend on split chains or the pipelined forward)
    char *fw = static_cast<char *>(const_cast<void *>(desc->forward_workspace));
    if (fw && !aligned(fw, 256)) return KDA_ERR_ALIGN;
    const bool fw_states = fw && desc->save_states == 1;  // the chunks' entering states too
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
    const WorkspaceLayout &fl = lay.fwd;
    int32_t *chunk_off = geo.varlen ? reinterpret_cast<int32_t *>(ws + fl.off_chunk_off) : nullptr;
    int32_t *seq_order = geo.varlen ? reinterpret_cast<int32_t *>(ws + fl.off_seq_order) : nullptr;
    hipEvent_t *ev = desc->phase_events;
    hipError_t err = hipSuccess;
    if (ev) err = hipEventRecord(ev[0], stream);
    if (err == hipSuccess && geo.varlen) err = kda_launch_chunk_table(cu_seqlens, geo.N, chunk_off, seq_order, stream);

    // the forward: intermediates, then the chain storing every chunk's entering state
    IntraArgs ia{};
    ia.q = static_cast<const uint16_t *>(q); ia.k = static_cast<const uint16_t *>(k);
    ia.v = static_cast<const uint16_t *>(v); ia.g = static_cast<const uint16_t *>(g);
    ia.beta = static_cast<const uint16_t *>(beta);
    ia.A_log = A_log; ia.dt_bias = dt_bias; ia.lower_bound = lower_bound;
    ia.cu = cu_seqlens; ia.chunk_off = chunk_off;
    ia.T = geo.T; ia.H = geo.H; ia.N = geo.N; ia.nc_fixed = geo.nc_fixed;
    char *fbase = fw ? fw : ws;
    ia.Wf = reinterpret_cast<_Float16 *>(fbase + fl.off_Wf);
    ia.Qf = reinterpret_cast<_Float16 *>(fbase + fl.off_Qf);
    ia.Kf = reinterpret_cast<_Float16 *>(fbase + fl.off_Kf);
    ia.Af = reinterpret_cast<_Float16 *>(fbase + fl.off_Af);
    ia.Uf = reinterpret_cast<_Float16 *>(fbase + fl.off_Uf);
    ia.gn = reinterpret_cast<float *>(fbase + fl.off_gn);
    ia.piece_cap = desc->launch_piece;
    if (err == hipSuccess && geo.T > 0 && !fw) err = kda_launch_intra(ia, geo.slots, stream);
    if (ev && err == hipSuccess) err = hipEventRecord(ev[1], stream);
    BwdArgs ba{};
    // the forward's states: from the kept workspace, past the end of its layout
    ba.hs = reinterpret_cast<float *>(fw_states ? fw + fl.total : ws + lay.off_hs);
    if (geo.T > 0 && !fw_states) {
        ChainArgs ca{};
        ca.Wf = ia.Wf; ca.Qf = ia.Qf; ca.Kf = ia.Kf; ca.Af = ia.Af; ca.Uf = ia.Uf; ca.gn = ia.gn;
        ca.cu = cu_seqlens; ca.chunk_off = chunk_off; ca.seq_order = seq_order;
        ca.T = geo.T; ca.H = geo.H; ca.N = geo.N; ca.nc_fixed = geo.nc_fixed;
        ca.scale = scale;
        ca.h0 = initial_state; ca.ht = nullptr;
        ca.h0_bf16 = desc->initial_state_dtype == KDA_BF16;
        ca.out = nullptr;  // the states only: save mode writes no outputs
        ca.hs = ba.hs;
        ca.piece_cap = desc->launch_piece;
        if (err == hipSuccess) err = launch_chains(ca, geo, fl, ws, stream);
    }
    if (ev && err == hipSuccess) err = hipEventRecord(ev[2], stream);
    // the gradient
    ba.q = ia.q; ba.k = ia.k; ba.v = ia.v; ba.g = ia.g; ba.beta = ia.beta;
    ba.A_log = A_log; ba.dt_bias = dt_bias; ba.lower_bound = lower_bound; ba.scale = scale;
    ba.dout = static_cast<const uint16_t *>(d_out);
    ba.dht = d_final_state; ba.dht_bf16 = desc->final_state_dtype == KDA_BF16;
    ba.cu = cu_seqlens; ba.chunk_off = chunk_off; ba.seq_order = seq_order;
    ba.T = geo.T; ba.H = geo.H; ba.N = geo.N; ba.nc_fixed = geo.nc_fixed;
    ba.slots = geo.T > 0 ? geo.slots : 0;
    ba.Wf = ia.Wf; ba.Qf = ia.Qf; ba.Kf = ia.Kf; ba.Af = ia.Af; ba.gn = ia.gn;
    ba.dhs = reinterpret_cast<float *>(ws + lay.off_dhs);
    ba.dUt = reinterpret_cast<float *>(ws + lay.off_dUt);
    ba.G = reinterpret_cast<float *>(ws + lay.off_G);
    ba.rq = reinterpret_cast<float *>(ws + lay.off_rq);
    ba.rk = reinterpret_cast<float *>(ws + lay.off_rk);
    ba.bb = reinterpret_cast<float *>(ws + lay.off_bb);
    ba.Mk = reinterpret_cast<float *>(ws + lay.off_Mk);
    ba.Tm = reinterpret_cast<float *>(ws + lay.off_Tm);
    ba.part = reinterpret_cast<float *>(ws + lay.off_part);
    ba.co = reinterpret_cast<unsigned char *>(ws + lay.off_co);
    ba.dq = dq; ba.dk = dk; ba.dv = dv; ba.dg = dg; ba.dbeta = dbeta;
    ba.dh0 = d_initial_state; ba.dA_log = dA_log; ba.ddt_bias = ddt_bias;
    ba.piece_cap = desc->launch_piece;
    if (err == hipSuccess) err = kda_launch_bwd_prep(ba, stream);
    if (ev && err == hipSuccess) err = hipEventRecord(ev[3], stream);
    if (err == hipSuccess) err = launch_bwd_chains(ba, geo, fl, ws, fw_states ? fw : ws, stream);
    if (ev && err == hipSuccess) err = hipEventRecord(ev[4], stream);
    if (err == hipSuccess) err = kda_launch_bwd_grad(ba, stream);
    if (ev && err == hipSuccess) err = hipEventRecord(ev[5], stream);
    if (owned) {
        hipError_t e2 = hipFreeAsync(ws, stream);
        if (err == hipSuccess) err = e2;
    }
    return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}
