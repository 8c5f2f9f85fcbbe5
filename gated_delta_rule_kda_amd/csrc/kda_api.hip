// C ABI of libkda (declared in include/kda.h): host-side validation, then the
// kernel launches.  Every check runs before anything is enqueued, so a call
// that returns an error has no side effects and needs no GPU to be tested.

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include "kda.h"
#include "kda_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

bool head_dim_ok(int d) { return d == 32 || d == 64 || d == 128; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A byte range [p, p + n) of one argument, for the overlap checks.
struct Range {
    const char *name;
    uintptr_t lo, hi;
};

Range rng(const char *name, const void *p, uint64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{name, lo, p ? lo + bytes : lo};
}

bool overlap(const Range &a, const Range &b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;  // empty or absent
    return a.lo < b.hi && b.lo < a.hi;
}

// Element count of a product of non-negative sizes; false on overflow past 2^50.
bool count(uint64_t &out, std::initializer_list<int64_t> dims) {
    uint64_t n = 1;
    for (int64_t d : dims) {
        if (d < 0) return false;
        if (d != 0 && n > (uint64_t(1) << 50) / static_cast<uint64_t>(d)) return false;
        n *= static_cast<uint64_t>(d);
    }
    out = n;
    return true;
}

__global__ void copy_or_zero_kernel(float *dst, const float *src, uint64_t n) {
    const uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char *kda_last_error(void) { return g_err; }

}  // extern "C"

namespace {

// Shared body of kda_chunk_fwd and kda_chunk_fwd_snapshots; `fn` names the
// entry point in error messages.
// The size checks shared by the prefill entry points and their workspace
// query: KDA_OK, or the code with the message set.
int prefill_sizes_ok(const char *fn, int B, int T, int H, int HV, int K, int V, int chunk,
                     int dtype) {
    if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16)
        return fail(KDA_EUNSUPPORTED, "%s: dtype %d is not KDA_DTYPE_F32 or KDA_DTYPE_BF16", fn, dtype);
    if (B < 0 || T < 0) return fail(KDA_EINVAL, "%s: B=%d and T=%d must be >= 0", fn, B, T);
    if (H < 1 || HV < 1) return fail(KDA_EINVAL, "%s: H=%d and HV=%d must be >= 1", fn, H, HV);
    if (HV % H != 0) return fail(KDA_EINVAL, "%s: HV=%d is not a multiple of H=%d", fn, HV, H);
    if (!head_dim_ok(K) || !head_dim_ok(V))
        return fail(KDA_EUNSUPPORTED, "%s: K=%d, V=%d; each must be 32, 64 or 128", fn, K, V);
    if (chunk < 0) return fail(KDA_EINVAL, "%s: chunk=%d must be >= 0", fn, chunk);
    if (chunk != 0 && chunk != 32)
        return fail(KDA_EUNSUPPORTED, "%s: chunk=%d; only 32 (or 0 for the default) is built", fn, chunk);
    return KDA_OK;
}

// Workspace bytes of a prefill call: the fused kernels keep every
// intermediate in registers and LDS, so none of the built paths needs any.
uint64_t prefill_workspace_bytes(int, int, int, int, int, int, int, int) { return 0; }

// Workspace bytes of kda_chunk_fwd_unbounded: every chunk's in-chunk matrices
// (kUnbImgElems bf16), [B, HV, NC]; sizes already validated.
uint64_t unbounded_workspace_bytes(int B, int T, int HV) {
    const uint64_t nc = (static_cast<uint64_t>(T) + 31) / 32;
    return static_cast<uint64_t>(B) * HV * nc * kda::kUnbImgElems * 2;
}

// Which kernels a prefill entry point runs.
enum class Path { chunk, recurrent, unbounded };

// The fused layer stages of kda_chunk_fwd_gated (none when A_log is NULL).
struct FusedStages {
    bool on = false;
    const float *A_log = nullptr, *dt_bias = nullptr;
    float lower_bound = 0.f;
    const void *ogate = nullptr;
    float og_eps = 0.f;
};

int chunk_fwd_impl(const char *fn, const void *q, const void *k, const void *v, const float *g,
                   const float *beta, const float *initial_state, void *out, float *final_state,
                   float *snapshots, int snapshot_every, int B, int T, int H, int HV, int K,
                   int V, float scale, int chunk, int dtype, void *workspace,
                   long long workspace_bytes, void *stream, Path path = Path::chunk,
                   const FusedStages &fs = FusedStages()) {
    g_err[0] = '\0';
    if (const int rc = prefill_sizes_ok(fn, B, T, H, HV, K, V, chunk, dtype)) return rc;
    if (path == Path::unbounded && dtype != KDA_DTYPE_BF16)
        return fail(KDA_EUNSUPPORTED, "%s: built for KDA_DTYPE_BF16 only (fp32 inputs: kda_recurrent_fwd)", fn);
    const bool fused = fs.on;
    if (fused) {
        if (dtype != KDA_DTYPE_BF16)
            return fail(KDA_EUNSUPPORTED, "%s: the fused stages are built for KDA_DTYPE_BF16 only", fn);
        if (!(fs.lower_bound >= -5.f && fs.lower_bound <= 0.f))
            return fail(KDA_EINVAL, "%s: gate_lower_bound=%g must lie in [-5, 0]", fn, fs.lower_bound);
        if (fs.ogate && !(fs.og_eps >= 0.f && isfinite(fs.og_eps)))
            return fail(KDA_EINVAL, "%s: out_gate_eps must be finite and >= 0", fn);
    }
    if (workspace_bytes < 0)
        return fail(KDA_EINVAL, "%s: workspace_bytes=%lld must be >= 0", fn, workspace_bytes);
    if (snapshots && (snapshot_every < 32 || snapshot_every % 32 != 0))
        return fail(KDA_EINVAL, "%s: snapshot_every=%d must be a positive multiple of the chunk size 32",
                    fn, snapshot_every);
    if (isinf(scale)) return fail(KDA_EINVAL, "%s: scale is infinite", fn);
    if (!(scale > 0.f)) scale = 1.0f / sqrtf(static_cast<float>(K));

    const uint64_t esz = dtype == KDA_DTYPE_BF16 ? 2 : 4;
    const int NS = snapshots ? T / snapshot_every : 0;
    uint64_t nq, nv, ng, nb, ns, nsn;
    if (!count(nq, {B, T, H, K}) || !count(nv, {B, T, HV, V}) || !count(ng, {B, T, HV, K}) ||
        !count(nb, {B, T, HV}) || !count(ns, {B, HV, K, V}) || !count(nsn, {B, NS, HV, K, V}))
        return fail(KDA_EINVAL, "%s: tensor sizes overflow", fn);
    const bool work = (static_cast<int64_t>(B) * T) > 0;
    const uint64_t ws_need = path == Path::recurrent ? 0
                             : path == Path::unbounded ? unbounded_workspace_bytes(B, T, HV)
                                                       : prefill_workspace_bytes(B, T, H, HV, K, V, chunk, dtype);
    if (work) {
        if (!q || !k || !v || !g || !beta || !out)
            return fail(KDA_EINVAL, "%s: q, k, v, %s, %s and out must be non-NULL", fn, fused ? "z" : "g",
                        fused ? "beta_logit" : "beta");
        if (fused && (!fs.A_log || !fs.dt_bias))
            return fail(KDA_EINVAL, "%s: A_log and dt_bias must be non-NULL", fn);
        if (ws_need > 0 && (!workspace || static_cast<uint64_t>(workspace_bytes) < ws_need))
            return fail(KDA_EINVAL, "%s: workspace of %lld bytes at %p, %llu needed", fn, workspace_bytes,
                        workspace, static_cast<unsigned long long>(ws_need));
    }
    // the workspace is only looked at when the call uses it
    const void *ws = work && ws_need > 0 ? workspace : nullptr;
    const void *ptrs[] = {q, k, v, g, beta, initial_state, out, final_state, snapshots, ws,
                          fs.A_log, fs.dt_bias, fs.ogate};
    const char *names[] = {"q", "k", "v", fused ? "z" : "g", fused ? "beta_logit" : "beta", "initial_state",
                           "out", "final_state", "snapshots", "workspace", "A_log", "dt_bias", "out_gate"};
    for (int i = 0; i < 13; ++i)
        if (ptrs[i] && !aligned16(ptrs[i]))
            return fail(KDA_EINVAL, "%s: %s is not 16-byte aligned", fn, names[i]);

    const Range r_in[] = {rng("q", q, nq * esz), rng("k", k, nq * esz), rng("v", v, nv * esz),
                          rng(fused ? "z" : "g", g, ng * 4), rng(fused ? "beta_logit" : "beta", beta, nb * 4),
                          rng("initial_state", initial_state, ns * 4),
                          rng("A_log", fs.A_log, static_cast<uint64_t>(HV) * 4),
                          rng("dt_bias", fs.dt_bias, static_cast<uint64_t>(HV) * K * 4),
                          rng("out_gate", fs.ogate, nv * esz)};
    const Range r_out = rng("out", out, nv * esz);
    const Range r_st = rng("final_state", final_state, ns * 4);
    for (const Range &r : r_in) {
        if (work && overlap(r_out, r)) return fail(KDA_EINVAL, "%s: out overlaps %s", fn, r.name);
        if (overlap(r_st, r) && !(&r == &r_in[5] && final_state == initial_state))
            return fail(KDA_EINVAL, "%s: final_state overlaps %s", fn, r.name);
    }
    if (work && overlap(r_out, r_st)) return fail(KDA_EINVAL, "%s: out overlaps final_state", fn);
    const Range r_sn = rng("snapshots", snapshots, nsn * 4);
    for (const Range &r : r_in)
        if (overlap(r_sn, r)) return fail(KDA_EINVAL, "%s: snapshots overlap %s", fn, r.name);
    if (overlap(r_sn, r_out) || overlap(r_sn, r_st))
        return fail(KDA_EINVAL, "%s: snapshots overlap %s", fn, overlap(r_sn, r_out) ? "out" : "final_state");
    const Range r_ws = rng("workspace", ws, ws_need);
    for (const Range &r : r_in)
        if (overlap(r_ws, r)) return fail(KDA_EINVAL, "%s: workspace overlaps %s", fn, r.name);
    if (overlap(r_ws, r_out) || overlap(r_ws, r_st) || overlap(r_ws, r_sn))
        return fail(KDA_EINVAL, "%s: workspace overlaps an output", fn);

    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!work) {
        // No tokens: the final state is the initial state (zeros when absent).
        if (final_state && final_state != initial_state && ns > 0) {
            const unsigned blocks = static_cast<unsigned>((ns + 255) / 256);
            hipLaunchKernelGGL(copy_or_zero_kernel, dim3(blocks), dim3(256), 0, st, final_state,
                               initial_state, ns);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return fail(KDA_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
        }
        return KDA_OK;
    }

    kda::PrefillArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.S0 = initial_state;
    a.out = out; a.ST = final_state;
    a.snap = NS > 0 ? snapshots : nullptr;
    a.snap_chunks = NS > 0 ? snapshot_every / 32 : 1;
    a.NS = NS;
    a.B = B; a.T = T; a.H = H; a.HV = HV; a.K = K; a.V = V;
    a.scale = scale;
    a.bf16 = dtype == KDA_DTYPE_BF16;
    a.A_log = fs.A_log; a.dt_bias = fs.dt_bias; a.lower_bound = fs.lower_bound;
    a.ogate = fs.ogate; a.og_eps = fs.og_eps;
    const hipError_t e = path == Path::recurrent ? kda::launch_recurrent(a, st)
                         : path == Path::unbounded
                             ? kda::launch_unbounded_prefill(a, static_cast<uint16_t *>(workspace), st)
                             : kda::launch_prefill(a, st);
    if (e != hipSuccess) return fail(KDA_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return KDA_OK;
}

}  // namespace

namespace {

// Workspace of kda_recurrent_bwd: fp32 regions, each 256-byte aligned (offsets
// in bytes).  The passes after the forward one run over slabs of Ls tokens
// (kBwdSlab, or all of T when shorter), so dr, the partial sums and the dg
// terms hold one slab; the forward residuals r cover the whole sequence, and
// the forward pass leaves the state at each later slab's start in snap.
struct BwdLayout {
    uint64_t r, dr, st, snap, Dc, daP, dqP, dkrP, e, bs, gc, total;
    int NCB, NB, Ls, NS;
};

bool bwd_layout(BwdLayout &L, int B, int T, int HV, int K, int V) {
    L.NCB = V / kda::kBwdCols;
    L.Ls = T < kda::kBwdSlab ? (T > 0 ? T : 1) : kda::kBwdSlab;
    L.NS = T > 0 ? (T - 1) / kda::kBwdSlab : 0;
    L.NB = (L.Ls + kda::kDgBlock - 1) / kda::kDgBlock;
    uint64_t nv, nvs, ns, nsn, np, ne, nbs, ngc;
    if (!count(nv, {B, T, HV, V}) || !count(nvs, {B, L.Ls, HV, V}) || !count(ns, {B, HV, K, V}) ||
        !count(nsn, {B, L.NS, HV, K, V}) || !count(np, {L.NCB, B, L.Ls, HV, K}) ||
        !count(ne, {B, L.Ls, HV, K}) || !count(nbs, {B, HV, L.NB, K}) || !count(ngc, {2, B, HV, K}))
        return false;
    uint64_t off = 0;
    auto take = [&](uint64_t floats) {
        const uint64_t at = off;
        off += (floats * 4 + 255) / 256 * 256;
        return at;
    };
    L.r = take(nv); L.dr = take(nvs); L.st = take(ns); L.snap = take(nsn); L.Dc = take(ns);
    L.daP = take(np); L.dqP = take(np); L.dkrP = take(np);
    L.e = take(ne); L.bs = take(nbs); L.gc = take(ngc);
    L.total = off;
    return true;
}

// Workspace of kda_chunk_bwd: fp32 regions, each 256-byte aligned (offsets in
// bytes).  Slabs of Ls tokens (1024, or T rounded up to the chunk when
// shorter); everything but the final state and the slab-start states holds one
// slab, and what one stream produces while another still reads the previous
// slab's (chunk-start states, U, operand images, dR, every chunk's dM') two,
// by slab parity.
struct ChunkBwdLayout {
    uint64_t st, snap1, Dc, snapc, U, img, snapc2, U2, img2, dR, dMs, dR2, dMs2, e, cs, gc, total;
    int Ls, NS1, NCs;
};

bool chunk_bwd_layout(ChunkBwdLayout &L, int B, int T, int HV, int K, int V) {
    L.Ls = T > kda::kBwdSlab ? kda::kBwdSlab : (T > 0 ? (T + 31) / 32 * 32 : 32);
    L.NS1 = T > 0 ? (T + L.Ls - 1) / L.Ls - 1 : 0;
    L.NCs = L.Ls / 32;
    const int imf = kda::chunk_bwd_image_floats(K);
    uint64_t ns, nsn, nsc, nv, nimg, nms, ne, ncs, ngc;
    if (imf <= 0 || !count(ns, {B, HV, K, V}) || !count(nsn, {B, L.NS1, HV, K, V}) ||
        !count(nsc, {B, L.NCs - 1, HV, K, V}) || !count(nv, {B, L.Ls, HV, V}) ||
        !count(nimg, {B, L.NCs, HV, imf}) || !count(nms, {B, L.NCs, HV, K, V}) ||
        !count(ne, {B, L.Ls, HV, K}) || !count(ncs, {B, HV, L.NCs, K}) || !count(ngc, {2, B, HV, K}))
        return false;
    uint64_t off = 0;
    auto take = [&](uint64_t floats) {
        const uint64_t at = off;
        off += (floats * 4 + 255) / 256 * 256;
        return at;
    };
    L.st = take(ns); L.snap1 = take(nsn); L.Dc = take(ns); L.snapc = take(nsc);
    L.U = take(nv); L.img = take(nimg);
    L.snapc2 = take(nsc); L.U2 = take(nv); L.img2 = take(nimg);
    L.dR = take(nv); L.dMs = take(nms);
    L.dR2 = take(nv); L.dMs2 = take(nms);
    L.e = take(ne); L.cs = take(ncs); L.gc = take(ngc);
    L.total = off;
    return true;
}

}  // namespace

extern "C" {

long long kda_chunk_fwd_workspace_size(int B, int T, int H, int HV, int K, int V, int chunk,
                                       int dtype) {
    g_err[0] = '\0';
    if (prefill_sizes_ok("kda_chunk_fwd_workspace_size", B, T, H, HV, K, V, chunk, dtype) != KDA_OK)
        return -1;
    uint64_t n;
    if (!count(n, {B, T, HV, K}) || !count(n, {B, T, HV, V})) {
        fail(KDA_EINVAL, "kda_chunk_fwd_workspace_size: tensor sizes overflow");
        return -1;
    }
    return static_cast<long long>(prefill_workspace_bytes(B, T, H, HV, K, V, chunk, dtype));
}

int kda_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                  const float *beta, const float *initial_state, void *out,
                  float *final_state, int B, int T, int H, int HV, int K, int V,
                  float scale, int chunk, int dtype, void *workspace,
                  long long workspace_bytes, void *stream) {
    return chunk_fwd_impl("kda_chunk_fwd", q, k, v, g, beta, initial_state, out, final_state,
                          nullptr, 0, B, T, H, HV, K, V, scale, chunk, dtype, workspace,
                          workspace_bytes, stream);
}

int kda_chunk_fwd_snapshots(const void *q, const void *k, const void *v, const float *g,
                            const float *beta, const float *initial_state, void *out,
                            float *final_state, float *snapshots, int snapshot_every,
                            int B, int T, int H, int HV, int K, int V, float scale,
                            int chunk, int dtype, void *workspace, long long workspace_bytes,
                            void *stream) {
    return chunk_fwd_impl("kda_chunk_fwd_snapshots", q, k, v, g, beta, initial_state, out,
                          final_state, snapshots, snapshot_every, B, T, H, HV, K, V, scale,
                          chunk, dtype, workspace, workspace_bytes, stream);
}

int kda_chunk_fwd_gated(const void *q, const void *k, const void *v, const float *z,
                        const float *beta_logit, const float *A_log, const float *dt_bias,
                        float gate_lower_bound, const float *initial_state, const void *out_gate,
                        float out_gate_eps, void *out, float *final_state, int B, int T, int H,
                        int HV, int K, int V, float scale, int chunk, int dtype, void *workspace,
                        long long workspace_bytes, void *stream) {
    FusedStages fs;
    fs.on = true;
    fs.A_log = A_log; fs.dt_bias = dt_bias; fs.lower_bound = gate_lower_bound;
    fs.ogate = out_gate; fs.og_eps = out_gate_eps;
    return chunk_fwd_impl("kda_chunk_fwd_gated", q, k, v, z, beta_logit, initial_state, out, final_state,
                          nullptr, 0, B, T, H, HV, K, V, scale, chunk, dtype, workspace, workspace_bytes,
                          stream, Path::chunk, fs);
}

int kda_recurrent_fwd(const void *q, const void *k, const void *v, const float *g,
                      const float *beta, const float *initial_state, void *out,
                      float *final_state, int B, int T, int H, int HV, int K, int V,
                      float scale, int dtype, void *stream) {
    return chunk_fwd_impl("kda_recurrent_fwd", q, k, v, g, beta, initial_state, out, final_state,
                          nullptr, 0, B, T, H, HV, K, V, scale, 0, dtype, nullptr, 0, stream, Path::recurrent);
}

long long kda_chunk_fwd_unbounded_workspace_size(int B, int T, int H, int HV, int K, int V, int dtype) {
    g_err[0] = '\0';
    const char *fn = "kda_chunk_fwd_unbounded_workspace_size";
    if (prefill_sizes_ok(fn, B, T, H, HV, K, V, 0, dtype) != KDA_OK) return -1;
    if (dtype != KDA_DTYPE_BF16) {
        fail(KDA_EUNSUPPORTED, "%s: built for KDA_DTYPE_BF16 only", fn);
        return -1;
    }
    uint64_t n;
    if (!count(n, {B, T, HV, K}) || !count(n, {B, T, HV, V}) || !count(n, {B, T / 32 + 1, HV, kda::kUnbImgElems})) {
        fail(KDA_EINVAL, "%s: tensor sizes overflow", fn);
        return -1;
    }
    return static_cast<long long>(unbounded_workspace_bytes(B, T, HV));
}

int kda_chunk_fwd_unbounded(const void *q, const void *k, const void *v, const float *g,
                            const float *beta, const float *initial_state, void *out,
                            float *final_state, int B, int T, int H, int HV, int K, int V,
                            float scale, int dtype, void *workspace, long long workspace_bytes,
                            void *stream) {
    return chunk_fwd_impl("kda_chunk_fwd_unbounded", q, k, v, g, beta, initial_state, out, final_state,
                          nullptr, 0, B, T, H, HV, K, V, scale, 0, dtype, workspace, workspace_bytes,
                          stream, Path::unbounded);
}

long long kda_recurrent_bwd_workspace_size(int B, int T, int H, int HV, int K, int V) {
    g_err[0] = '\0';
    if (B < 0 || T < 0 || H < 1 || HV < 1 || HV % H != 0) {
        fail(KDA_EINVAL, "kda_recurrent_bwd_workspace_size: B=%d, T=%d, H=%d, HV=%d are not valid sizes",
             B, T, H, HV);
        return -1;
    }
    if (!head_dim_ok(K) || !head_dim_ok(V)) {
        fail(KDA_EUNSUPPORTED, "kda_recurrent_bwd_workspace_size: K=%d, V=%d; each must be 32, 64 or 128", K, V);
        return -1;
    }
    BwdLayout L;
    if (!bwd_layout(L, B, T, HV, K, V)) {
        fail(KDA_EINVAL, "kda_recurrent_bwd_workspace_size: tensor sizes overflow");
        return -1;
    }
    return static_cast<long long>(L.total);
}

long long kda_chunk_bwd_workspace_size(int B, int T, int H, int HV, int K, int V, int dtype) {
    g_err[0] = '\0';
    const char *fn = "kda_chunk_bwd_workspace_size";
    if (dtype != KDA_DTYPE_BF16) {
        fail(KDA_EUNSUPPORTED, "%s: dtype %d; the chunked backward takes KDA_DTYPE_BF16 (use kda_recurrent_bwd)", fn, dtype);
        return -1;
    }
    if (B < 0 || T < 0 || H < 1 || HV < 1 || HV % H != 0) {
        fail(KDA_EINVAL, "%s: B=%d, T=%d, H=%d, HV=%d are not valid sizes", fn, B, T, H, HV);
        return -1;
    }
    if (!head_dim_ok(K) || !head_dim_ok(V)) {
        fail(KDA_EUNSUPPORTED, "%s: K=%d, V=%d; each must be 32, 64 or 128", fn, K, V);
        return -1;
    }
    ChunkBwdLayout L;
    if (!chunk_bwd_layout(L, B, T, HV, K, V)) {
        fail(KDA_EINVAL, "%s: tensor sizes overflow", fn);
        return -1;
    }
    return static_cast<long long>(L.total);
}

}  // extern "C"

namespace {

// Shared body of kda_chunk_bwd and kda_chunk_bwd_saved (saved: the forward's
// states every kBwdSlab tokens and its final state come from the caller).
int chunk_bwd_impl(const char *fn, bool saved, const void *q, const void *k, const void *v, const float *g,
                   const float *beta, const float *initial_state, const float *saved_states,
                   const float *final_state, const void *dout, const float *dfinal_state, void *dq, void *dk,
                   void *dv, float *dg, float *dbeta, float *dinitial_state, int B, int T, int H, int HV, int K,
                   int V, float scale, int dtype, void *workspace, long long workspace_bytes, void *stream) {
    g_err[0] = '\0';
    if (dtype != KDA_DTYPE_BF16)
        return fail(KDA_EUNSUPPORTED, "%s: dtype %d; the chunked backward takes KDA_DTYPE_BF16 (use kda_recurrent_bwd)", fn, dtype);
    if (B < 0 || T < 0) return fail(KDA_EINVAL, "%s: B=%d and T=%d must be >= 0", fn, B, T);
    if (H < 1 || HV < 1) return fail(KDA_EINVAL, "%s: H=%d and HV=%d must be >= 1", fn, H, HV);
    if (HV % H != 0) return fail(KDA_EINVAL, "%s: HV=%d is not a multiple of H=%d", fn, HV, H);
    if (!head_dim_ok(K) || !head_dim_ok(V))
        return fail(KDA_EUNSUPPORTED, "%s: K=%d, V=%d; each must be 32, 64 or 128", fn, K, V);
    if (static_cast<int64_t>(B) * HV * 32 > 0x7fffffffLL)
        return fail(KDA_EUNSUPPORTED, "%s: B=%d, HV=%d exceed the launch grid", fn, B, HV);
    if (isinf(scale)) return fail(KDA_EINVAL, "%s: scale is infinite", fn);
    if (!(scale > 0.f)) scale = 1.0f / sqrtf(static_cast<float>(K));
    ChunkBwdLayout L;
    const int NSs = saved ? T / kda::kBwdSlab : 0;
    uint64_t nq, nv, ng, nb, ns, nss;
    if (!chunk_bwd_layout(L, B, T, HV, K, V) || !count(nq, {B, T, H, K}) || !count(nv, {B, T, HV, V}) ||
        !count(ng, {B, T, HV, K}) || !count(nb, {B, T, HV}) || !count(ns, {B, HV, K, V}) ||
        !count(nss, {B, NSs, HV, K, V}))
        return fail(KDA_EINVAL, "%s: tensor sizes overflow", fn);
    const bool work = static_cast<int64_t>(B) * T > 0;
    if (work) {
        if (!q || !k || !v || !g || !beta || !dout)
            return fail(KDA_EINVAL, "%s: q, k, v, g, beta and dout must be non-NULL", fn);
        if (!dq || !dk || !dv || !dg || !dbeta)
            return fail(KDA_EINVAL, "%s: dq, dk, dv, dg and dbeta must be non-NULL", fn);
        if (saved && L.NS1 > 0 && !saved_states)
            return fail(KDA_EINVAL, "%s: saved_states must be non-NULL when T > %d", fn, kda::kBwdSlab);
        if (saved && dfinal_state && !final_state)
            return fail(KDA_EINVAL, "%s: final_state must be non-NULL when dfinal_state is given", fn);
        if (!workspace) return fail(KDA_EINVAL, "%s: workspace is NULL", fn);
        if (workspace_bytes < 0 || static_cast<uint64_t>(workspace_bytes) < L.total)
            return fail(KDA_EINVAL, "%s: workspace of %lld bytes, %llu needed", fn, workspace_bytes,
                        static_cast<unsigned long long>(L.total));
    }
    const void *ptrs[] = {q, k, v, g, beta, initial_state, dout, dfinal_state, saved_states, final_state,
                          dq, dk, dv, dg, dbeta, dinitial_state, workspace};
    const char *names[] = {"q", "k", "v", "g", "beta", "initial_state", "dout", "dfinal_state",
                           "saved_states", "final_state", "dq", "dk", "dv", "dg", "dbeta", "dinitial_state",
                           "workspace"};
    for (int i = 0; i < 17; ++i)
        if (ptrs[i] && !aligned16(ptrs[i]))
            return fail(KDA_EINVAL, "%s: %s is not 16-byte aligned", fn, names[i]);
    const Range rs[] = {rng("q", q, nq * 2), rng("k", k, nq * 2), rng("v", v, nv * 2),
                        rng("g", g, ng * 4), rng("beta", beta, nb * 4),
                        rng("initial_state", initial_state, ns * 4), rng("dout", dout, nv * 2),
                        rng("dfinal_state", dfinal_state, ns * 4),
                        rng("saved_states", saved ? saved_states : nullptr, nss * 4),
                        rng("final_state", saved ? final_state : nullptr, ns * 4),
                        rng("dq", dq, nq * 2), rng("dk", dk, nq * 2), rng("dv", dv, nv * 2),
                        rng("dg", dg, ng * 4), rng("dbeta", dbeta, nb * 4),
                        rng("dinitial_state", dinitial_state, ns * 4),
                        rng("workspace", work ? workspace : nullptr, L.total)};
    for (int o = 10; o < 17; ++o)
        for (int i = 0; i < 17; ++i)
            if (i != o && overlap(rs[o], rs[i]))
                return fail(KDA_EINVAL, "%s: %s overlaps %s", fn, rs[o].name, rs[i].name);

    char *ws = static_cast<char *>(workspace);
    kda::ChunkBwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.S0 = initial_state;
    a.dout = dout; a.dST = dfinal_state;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.dS0 = dinitial_state;
    if (work) {
        auto at = [&](uint64_t off) { return reinterpret_cast<float *>(ws + off); };
        a.ST = at(L.st); a.snap1 = at(L.snap1); a.Dc = at(L.Dc); a.snapc = at(L.snapc);
        a.U = at(L.U); a.img = at(L.img); a.dR = at(L.dR); a.dMs = at(L.dMs);
        a.snapc2 = at(L.snapc2); a.U2 = at(L.U2); a.img2 = at(L.img2);
        a.dR2 = at(L.dR2); a.dMs2 = at(L.dMs2);
        a.e = at(L.e); a.cs = at(L.cs); a.gc = at(L.gc);
        if (saved) {
            // read only: the kernels never write ST or snap1 in this variant
            a.ST = const_cast<float *>(final_state);
            a.snap1 = const_cast<float *>(saved_states);
        }
    }
    a.saved = saved;
    a.NSsaved = NSs;
    a.Ls = L.Ls; a.NS1 = L.NS1;
    a.B = B; a.T = T; a.H = H; a.HV = HV; a.K = K; a.V = V;
    a.scale = scale;
    const hipError_t e = kda::launch_chunk_backward(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KDA_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return KDA_OK;
}

}  // namespace

extern "C" {

int kda_chunk_bwd(const void *q, const void *k, const void *v, const float *g, const float *beta,
                  const float *initial_state, const void *dout, const float *dfinal_state, void *dq,
                  void *dk, void *dv, float *dg, float *dbeta, float *dinitial_state, int B, int T,
                  int H, int HV, int K, int V, float scale, int dtype, void *workspace,
                  long long workspace_bytes, void *stream) {
    return chunk_bwd_impl("kda_chunk_bwd", false, q, k, v, g, beta, initial_state, nullptr, nullptr, dout,
                          dfinal_state, dq, dk, dv, dg, dbeta, dinitial_state, B, T, H, HV, K, V, scale, dtype,
                          workspace, workspace_bytes, stream);
}

int kda_chunk_bwd_saved(const void *q, const void *k, const void *v, const float *g, const float *beta,
                        const float *initial_state, const float *saved_states, const float *final_state,
                        const void *dout, const float *dfinal_state, void *dq, void *dk, void *dv, float *dg,
                        float *dbeta, float *dinitial_state, int B, int T, int H, int HV, int K, int V,
                        float scale, int dtype, void *workspace, long long workspace_bytes, void *stream) {
    return chunk_bwd_impl("kda_chunk_bwd_saved", true, q, k, v, g, beta, initial_state, saved_states,
                          final_state, dout, dfinal_state, dq, dk, dv, dg, dbeta, dinitial_state, B, T, H, HV, K,
                          V, scale, dtype, workspace, workspace_bytes, stream);
}

}  // extern "C"

// Scratch for kda_recurrent_bwd_noalloc: in the code object's device memory,
// one copy per GPU the library runs on, held until the process ends.  Host
// code never uses this name as an address (on the host it is a stand-in
// symbol); the device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the GPU `stream` runs on (the current
// device for the NULL stream), looked up once per device with that device
// current.
int scratch_for_stream(const char *fn, hipStream_t stream, void **out) {
    int cur = -1, dev = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return fail(KDA_EHIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    dev = cur;
    if (stream) {
        e = hipStreamGetDevice(stream, &dev);
        if (e != hipSuccess) return fail(KDA_EHIP, "%s: hipStreamGetDevice: %s", fn, hipGetErrorString(e));
    }
    if (dev < 0 || dev >= kMaxDevices)
        return fail(KDA_EUNSUPPORTED, "%s: device %d; devices 0..%d are supported", fn, dev, kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
            return fail(KDA_EHIP, "%s: hipSetDevice(%d): %s", fn, dev, hipGetErrorString(e));
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t e2 = dev != cur ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess)
            return fail(KDA_EHIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                        hipGetErrorString(e));
        if (e2 != hipSuccess) return fail(KDA_EHIP, "%s: hipSetDevice(%d): %s", fn, cur, hipGetErrorString(e2));
        if (!p || !aligned16(p)) return fail(KDA_EHIP, "%s: scratch address %p on device %d", fn, p, dev);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KDA_OK;
}

// Shared body of kda_recurrent_bwd and kda_recurrent_bwd_noalloc (noalloc:
// the workspace arguments are ignored and the device's scratch array serves
// instead, once the arguments have passed validation).
int recurrent_bwd_impl(const char *fn, const void *q, const void *k, const void *v, const float *g,
                       const float *beta, const float *initial_state, const void *dout,
                       const float *dfinal_state, void *dq, void *dk, void *dv, float *dg,
                       float *dbeta, float *dinitial_state, int B, int T, int H, int HV, int K,
                       int V, float scale, int dtype, void *workspace, long long workspace_bytes,
                       void *stream, bool noalloc) {
    g_err[0] = '\0';
    if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16)
        return fail(KDA_EUNSUPPORTED, "%s: dtype %d is not KDA_DTYPE_F32 or KDA_DTYPE_BF16", fn, dtype);
    if (B < 0 || T < 0) return fail(KDA_EINVAL, "%s: B=%d and T=%d must be >= 0", fn, B, T);
    if (H < 1 || HV < 1) return fail(KDA_EINVAL, "%s: H=%d and HV=%d must be >= 1", fn, H, HV);
    if (HV % H != 0) return fail(KDA_EINVAL, "%s: HV=%d is not a multiple of H=%d", fn, HV, H);
    if (!head_dim_ok(K) || !head_dim_ok(V))
        return fail(KDA_EUNSUPPORTED, "%s: K=%d, V=%d; each must be 32, 64 or 128", fn, K, V);
    if (isinf(scale)) return fail(KDA_EINVAL, "%s: scale is infinite", fn);
    if (!(scale > 0.f)) scale = 1.0f / sqrtf(static_cast<float>(K));
    BwdLayout L;
    uint64_t nq, nv, ng, nb, ns;
    if (!bwd_layout(L, B, T, HV, K, V) || !count(nq, {B, T, H, K}) || !count(nv, {B, T, HV, V}) ||
        !count(ng, {B, T, HV, K}) || !count(nb, {B, T, HV}) || !count(ns, {B, HV, K, V}))
        return fail(KDA_EINVAL, "%s: tensor sizes overflow", fn);
    const uint64_t esz = dtype == KDA_DTYPE_BF16 ? 2 : 4;
    const bool work = static_cast<int64_t>(B) * T > 0;
    if (work) {
        if (!q || !k || !v || !g || !beta || !dout)
            return fail(KDA_EINVAL, "%s: q, k, v, g, beta and dout must be non-NULL", fn);
        if (!dq || !dk || !dv || !dg || !dbeta)
            return fail(KDA_EINVAL, "%s: dq, dk, dv, dg and dbeta must be non-NULL", fn);
        if (noalloc) {
            if (L.total > KDA_NOALLOC_SCRATCH_BYTES)
                return fail(KDA_EUNSUPPORTED,
                            "%s: these sizes need %llu bytes of scratch, more than the %llu bytes of the "
                            "library's array (use kda_recurrent_bwd with a workspace)",
                            fn, static_cast<unsigned long long>(L.total),
                            static_cast<unsigned long long>(KDA_NOALLOC_SCRATCH_BYTES));
            workspace = nullptr;   // not a caller buffer: set below, after validation
        } else {
            if (!workspace) return fail(KDA_EINVAL, "%s: workspace is NULL", fn);
            if (workspace_bytes < 0 || static_cast<uint64_t>(workspace_bytes) < L.total)
                return fail(KDA_EINVAL, "%s: workspace of %lld bytes, %llu needed", fn, workspace_bytes,
                            static_cast<unsigned long long>(L.total));
        }
    }
    const void *ptrs[] = {q, k, v, g, beta, initial_state, dout, dfinal_state,
                          dq, dk, dv, dg, dbeta, dinitial_state, workspace};
    const char *names[] = {"q", "k", "v", "g", "beta", "initial_state", "dout", "dfinal_state",
                           "dq", "dk", "dv", "dg", "dbeta", "dinitial_state", "workspace"};
    for (int i = 0; i < 15; ++i)
        if (ptrs[i] && !aligned16(ptrs[i]))
            return fail(KDA_EINVAL, "%s: %s is not 16-byte aligned", fn, names[i]);
    // every output (and the workspace) is disjoint from every other argument
    const Range rs[] = {rng("q", q, nq * esz), rng("k", k, nq * esz), rng("v", v, nv * esz),
                        rng("g", g, ng * 4), rng("beta", beta, nb * 4),
                        rng("initial_state", initial_state, ns * 4), rng("dout", dout, nv * esz),
                        rng("dfinal_state", dfinal_state, ns * 4),
                        rng("dq", dq, nq * esz), rng("dk", dk, nq * esz), rng("dv", dv, nv * esz),
                        rng("dg", dg, ng * 4), rng("dbeta", dbeta, nb * 4),
                        rng("dinitial_state", dinitial_state, ns * 4),
                        rng("workspace", work ? workspace : nullptr, L.total)};
    for (int o = 8; o < 15; ++o)
        for (int i = 0; i < 15; ++i)
            if (i != o && overlap(rs[o], rs[i]))
                return fail(KDA_EINVAL, "%s: %s overlaps %s", fn, rs[o].name, rs[i].name);

    hipStream_t st = static_cast<hipStream_t>(stream);
    if (noalloc && work) {
        if (const int rc = scratch_for_stream(fn, st, &workspace)) return rc;
    }
    char *ws = static_cast<char *>(workspace);
    kda::BwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.S0 = initial_state;
    a.dout = dout; a.dST = dfinal_state;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.dS0 = dinitial_state;
    if (work) {
        a.r = reinterpret_cast<float *>(ws + L.r);
        a.dr = reinterpret_cast<float *>(ws + L.dr);
        a.ST = reinterpret_cast<float *>(ws + L.st);
        a.daP = reinterpret_cast<float *>(ws + L.daP);
        a.dqP = reinterpret_cast<float *>(ws + L.dqP);
        a.dkrP = reinterpret_cast<float *>(ws + L.dkrP);
        a.e = reinterpret_cast<float *>(ws + L.e);
        a.bs = reinterpret_cast<float *>(ws + L.bs);
        a.snap = reinterpret_cast<float *>(ws + L.snap);
        a.Dc = reinterpret_cast<float *>(ws + L.Dc);
        a.gc_in = reinterpret_cast<float *>(ws + L.gc);
        a.gc_out = reinterpret_cast<float *>(ws + L.gc) + static_cast<size_t>(B) * HV * K;
    }
    a.NCB = L.NCB; a.NB = L.NB; a.Ls = L.Ls; a.NS = L.NS;
    a.B = B; a.T = T; a.H = H; a.HV = HV; a.K = K; a.V = V;
    a.scale = scale;
    a.bf16 = dtype == KDA_DTYPE_BF16;
    if (work) {
        // the forward pass, keeping the residuals and the final state
        kda::PrefillArgs f{};
        f.q = q; f.k = k; f.v = v; f.g = g; f.beta = beta; f.S0 = initial_state;
        f.out = nullptr; f.ST = a.ST; f.aux = a.r;
        // the states at the later slabs' starts, for the forward gradient pass
        f.snap = L.NS > 0 ? const_cast<float *>(a.snap) : nullptr;
        f.snap_chunks = kda::kBwdSlab / 32; f.NS = L.NS;
        f.B = B; f.T = T; f.H = H; f.HV = HV; f.K = K; f.V = V;
        f.scale = scale; f.bf16 = a.bf16;
        const hipError_t e = kda::launch_recurrent(f, st);
        if (e != hipSuccess) return fail(KDA_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    } else if (!dinitial_state || B == 0) {
        return KDA_OK;
    }
    const hipError_t e = kda::launch_backward(a, st);
    if (e != hipSuccess) return fail(KDA_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return KDA_OK;
}

}  // namespace

extern "C" {

int kda_recurrent_bwd(const void *q, const void *k, const void *v, const float *g,
                      const float *beta, const float *initial_state, const void *dout,
                      const float *dfinal_state, void *dq, void *dk, void *dv, float *dg,
                      float *dbeta, float *dinitial_state, int B, int T, int H, int HV, int K,
                      int V, float scale, int dtype, void *workspace, long long workspace_bytes,
                      void *stream) {
    return recurrent_bwd_impl("kda_recurrent_bwd", q, k, v, g, beta, initial_state, dout, dfinal_state,
                              dq, dk, dv, dg, dbeta, dinitial_state, B, T, H, HV, K, V, scale, dtype,
                              workspace, workspace_bytes, stream, false);
}

int kda_recurrent_bwd_noalloc(const void *q, const void *k, const void *v, const float *g,
                              const float *beta, const float *initial_state, const void *dout,
                              const float *dfinal_state, void *dq, void *dk, void *dv, float *dg,
                              float *dbeta, float *dinitial_state, int B, int T, int H, int HV,
                              int K, int V, float scale, int dtype, void *stream) {
    return recurrent_bwd_impl("kda_recurrent_bwd_noalloc", q, k, v, g, beta, initial_state, dout,
                              dfinal_state, dq, dk, dv, dg, dbeta, dinitial_state, B, T, H, HV, K, V,
                              scale, dtype, nullptr, 0, stream, true);
}

int kda_prefill_prologue(const void *x, const float *gate, const float *beta,
                         const kda_decode_prologue *pro, void *q, void *k, void *v,
                         float *g, float *beta_out, int B, int T, int H, int HV, int K,
                         int V, int dtype, void *stream) {
    g_err[0] = '\0';
    const char *fn = "kda_prefill_prologue";
    if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16)
        return fail(KDA_EUNSUPPORTED, "%s: dtype %d is not KDA_DTYPE_F32 or KDA_DTYPE_BF16", fn, dtype);
    if (B < 0 || T < 0) return fail(KDA_EINVAL, "%s: B=%d and T=%d must be >= 0", fn, B, T);
    if (H < 1 || HV < 1) return fail(KDA_EINVAL, "%s: H=%d and HV=%d must be >= 1", fn, H, HV);
    if (HV % H != 0) return fail(KDA_EINVAL, "%s: HV=%d is not a multiple of H=%d", fn, HV, H);
    if (!head_dim_ok(K) || !head_dim_ok(V))
        return fail(KDA_EUNSUPPORTED, "%s: K=%d, V=%d; each must be 32, 64 or 128", fn, K, V);
    if (B > 65535 || T > 65535 * 256)
        return fail(KDA_EUNSUPPORTED, "%s: B=%d must be <= 65535 and T=%d <= 16776960", fn, B, T);
    kda_decode_prologue p{};
    if (pro) p = *pro;
    const bool conv = p.conv_weight != nullptr;
    if (conv) {
        if (p.conv_kernel < 1) return fail(KDA_EINVAL, "%s: conv_kernel=%d must be >= 1", fn, p.conv_kernel);
        if (p.conv_kernel > 8)
            return fail(KDA_EUNSUPPORTED, "%s: conv_kernel=%d; at most 8 is built", fn, p.conv_kernel);
        if (p.conv_ring && (p.conv_pos < 0 || p.conv_pos >= p.conv_kernel))
            return fail(KDA_EINVAL, "%s: conv_pos=%d must be in 0..conv_kernel-1=%d", fn, p.conv_pos,
                        p.conv_kernel - 1);
    }
    if (p.gate_mode < 0 || p.gate_mode > 2)
        return fail(KDA_EINVAL, "%s: gate_mode=%d is not a kda_gate_mode", fn, p.gate_mode);
    if (p.gate_mode != KDA_GATE_DIRECT && (g || beta_out) && (!p.A_log || !p.dt_bias))
        return fail(KDA_EINVAL, "%s: gate_mode %d needs A_log and dt_bias", fn, p.gate_mode);
    if (p.l2norm_qk && !(p.l2_eps >= 0.f && isfinite(p.l2_eps)))
        return fail(KDA_EINVAL, "%s: l2_eps must be finite and >= 0", fn);

    const uint64_t esz = dtype == KDA_DTYPE_BF16 ? 2 : 4;
    const int64_t C = 2 * static_cast<int64_t>(H) * K + static_cast<int64_t>(HV) * V;
    const int KW = conv ? p.conv_kernel : 0;
    uint64_t nx, nq, nv, ng, nb, ncs, ncw, nal, ndt;
    if (!count(nx, {B, T, C}) || !count(nq, {B, T, H, K}) || !count(nv, {B, T, HV, V}) ||
        !count(ng, {B, T, HV, K}) || !count(nb, {B, T, HV}) || !count(ncs, {B, C, KW}) ||
        !count(ncw, {C, KW}) || !count(nal, {HV}) || !count(ndt, {HV, K}) || nx >= (uint64_t(1) << 40))
        return fail(KDA_EINVAL, "%s: tensor sizes overflow", fn);
    if (static_cast<int64_t>(B) * T == 0) return KDA_OK;
    // g and beta_out both NULL: no gate or beta stage (kda_chunk_fwd_gated
    // forms them itself); gate and beta are then not read
    const bool gate_stage = g || beta_out;
    if (!x || !q || !k || !v) return fail(KDA_EINVAL, "%s: x, q, k and v must be non-NULL", fn);
    if (gate_stage && (!gate || !beta || !g || !beta_out))
        return fail(KDA_EINVAL, "%s: gate, beta, g and beta_out must be non-NULL (or g and beta_out both NULL)", fn);
    if (!gate_stage) {
        gate = nullptr;
        beta = nullptr;
    }
    const void *ptrs[] = {x, gate, beta, q, k, v, g, beta_out, p.conv_weight, p.conv_state, p.A_log, p.dt_bias};
    const char *names[] = {"x", "gate", "beta", "q", "k", "v", "g", "beta_out", "conv_weight", "conv_state",
                           "A_log", "dt_bias"};
    for (int i = 0; i < 12; ++i)
        if (ptrs[i] && !aligned16(ptrs[i]))
            return fail(KDA_EINVAL, "%s: %s is not 16-byte aligned", fn, names[i]);
    const bool gp = gate_stage && p.gate_mode != KDA_GATE_DIRECT;
    const Range rs[] = {rng("x", x, nx * esz), rng("gate", gate, ng * 4), rng("beta", beta, nb * 4),
                        rng("q", q, nq * esz), rng("k", k, nq * esz), rng("v", v, nv * esz),
                        rng("g", g, ng * 4), rng("beta_out", beta_out, nb * 4),
                        rng("conv_weight", p.conv_weight, ncw * 4),
                        rng("conv_state", conv ? p.conv_state : nullptr, ncs * 4),
                        rng("A_log", gp ? p.A_log : nullptr, nal * 4),
                        rng("dt_bias", gp ? p.dt_bias : nullptr, ndt * 4)};
    const int outs[] = {3, 4, 5, 6, 7, 9};
    for (int o : outs)
        for (int i = 0; i < 12; ++i)
            if (i != o && overlap(rs[o], rs[i]))
                return fail(KDA_EINVAL, "%s: %s overlaps %s", fn, rs[o].name, rs[i].name);

    kda::PrologueArgs a{};
    a.x = x; a.conv_w = conv ? p.conv_weight : nullptr;
    a.conv_state = conv ? p.conv_state : nullptr;
    a.conv_state_out = conv ? p.conv_state : nullptr;
    a.KW = KW; a.l2norm = p.l2norm_qk ? 1 : 0; a.l2_eps = p.l2_eps;
    a.conv_ring = conv && p.conv_ring ? 1 : 0; a.conv_pos = a.conv_ring ? p.conv_pos : 0;
    a.gate = gate; a.gate_mode = p.gate_mode; a.A_log = p.A_log; a.dt_bias = p.dt_bias;
    a.lower_bound = p.gate_lower_bound; a.beta_in = beta; a.beta_is_logit = p.beta_is_logit ? 1 : 0;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta_out = beta_out;
    a.B = B; a.T = T; a.H = H; a.HV = HV; a.K = K; a.V = V;
    a.bf16 = dtype == KDA_DTYPE_BF16;
    const hipError_t e = kda::launch_prologue(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KDA_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return KDA_OK;
}

int kda_output_gate(const void *o, const void *gate, void *y, long long rows, int head_dim,
                    float eps, int dtype, void *stream) {
    g_err[0] = '\0';
    const char *fn = "kda_output_gate";
    if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16)
        return fail(KDA_EUNSUPPORTED, "%s: dtype %d is not KDA_DTYPE_F32 or KDA_DTYPE_BF16", fn, dtype);
    if (rows < 0) return fail(KDA_EINVAL, "%s: rows=%lld must be >= 0", fn, rows);
    if (!head_dim_ok(head_dim))
        return fail(KDA_EUNSUPPORTED, "%s: head_dim=%d must be 32, 64 or 128", fn, head_dim);
    if (!(eps >= 0.f && isfinite(eps))) return fail(KDA_EINVAL, "%s: eps must be finite and >= 0", fn);
    if (rows > (int64_t(1) << 40) / head_dim) return fail(KDA_EINVAL, "%s: tensor sizes overflow", fn);
    if (rows == 0) return KDA_OK;
    if (!o || !gate || !y) return fail(KDA_EINVAL, "%s: o, gate and y must be non-NULL", fn);
    const void *ptrs[] = {o, gate, y};
    const char *names[] = {"o", "gate", "y"};
    for (int i = 0; i < 3; ++i)
        if (!aligned16(ptrs[i])) return fail(KDA_EINVAL, "%s: %s is not 16-byte aligned", fn, names[i]);
    const uint64_t n = static_cast<uint64_t>(rows) * head_dim * (dtype == KDA_DTYPE_BF16 ? 2 : 4);
    const Range ro = rng("o", o, n), rg = rng("gate", gate, n), ry = rng("y", y, n);
    if (overlap(ry, rg)) return fail(KDA_EINVAL, "%s: y overlaps gate", fn);
    if (y != o && overlap(ry, ro)) return fail(KDA_EINVAL, "%s: y overlaps o (only y == o is allowed)", fn);

    kda::OutputGateArgs a{};
    a.o = o; a.gate = gate; a.y = y; a.rows = static_cast<long>(rows); a.D = head_dim; a.eps = eps;
    a.bf16 = dtype == KDA_DTYPE_BF16;
    const hipError_t e = kda::launch_output_gate(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KDA_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return KDA_OK;
}

int kda_decode_step(const void *qkv, const float *gate, const float *beta, float *state,
                    void *out, const kda_decode_prologue *pro, int B, int H, int HV, int K,
                    int V, float scale, int dtype, void *stream) {
    g_err[0] = '\0';
    if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16)
        return fail(KDA_EUNSUPPORTED, "kda_decode_step: dtype %d is not KDA_DTYPE_F32 or KDA_DTYPE_BF16", dtype);
    if (B < 0) return fail(KDA_EINVAL, "kda_decode_step: B=%d must be >= 0", B);
    if (H < 1 || HV < 1) return fail(KDA_EINVAL, "kda_decode_step: H=%d and HV=%d must be >= 1", H, HV);
    if (HV % H != 0) return fail(KDA_EINVAL, "kda_decode_step: HV=%d is not a multiple of H=%d", HV, H);
    if (!head_dim_ok(K) || !head_dim_ok(V))
        return fail(KDA_EUNSUPPORTED, "kda_decode_step: K=%d, V=%d; each must be 32, 64 or 128", K, V);
    if (isinf(scale)) return fail(KDA_EINVAL, "kda_decode_step: scale is infinite");
    if (!(scale > 0.f)) scale = 1.0f / sqrtf(static_cast<float>(K));

    kda_decode_prologue p{};
    if (pro) p = *pro;
    const bool conv = p.conv_weight != nullptr;
    if (conv) {
        if (!p.conv_state) return fail(KDA_EINVAL, "kda_decode_step: conv_weight given without conv_state");
        if (p.conv_kernel < 1) return fail(KDA_EINVAL, "kda_decode_step: conv_kernel=%d must be >= 1", p.conv_kernel);
        if (p.conv_kernel > 8)
            return fail(KDA_EUNSUPPORTED, "kda_decode_step: conv_kernel=%d; at most 8 is built", p.conv_kernel);
        if (p.conv_ring && (p.conv_pos < 0 || p.conv_pos >= p.conv_kernel))
            return fail(KDA_EINVAL, "kda_decode_step: conv_pos=%d must be in 0..conv_kernel-1=%d", p.conv_pos,
                        p.conv_kernel - 1);
    }
    if (p.gate_mode < 0 || p.gate_mode > 2)
        return fail(KDA_EINVAL, "kda_decode_step: gate_mode=%d is not a kda_gate_mode", p.gate_mode);
    if (p.gate_mode != KDA_GATE_DIRECT && (!p.A_log || !p.dt_bias))
        return fail(KDA_EINVAL, "kda_decode_step: gate_mode %d needs A_log and dt_bias", p.gate_mode);
    if (p.l2norm_qk && !(p.l2_eps >= 0.f && isfinite(p.l2_eps)))
        return fail(KDA_EINVAL, "kda_decode_step: l2_eps must be finite and >= 0");

    const uint64_t esz = dtype == KDA_DTYPE_BF16 ? 2 : 4;
    const int64_t C = 2 * static_cast<int64_t>(H) * K + static_cast<int64_t>(HV) * V;
    uint64_t nx, ng, nb, ns, no, ncs, ncw, nal, ndt;
    if (!count(nx, {B, C}) || !count(ng, {B, HV, K}) || !count(nb, {B, HV}) ||
        !count(ns, {B, HV, K, V}) || !count(no, {B, HV, V}) ||
        !count(ncs, {B, C, conv ? p.conv_kernel : 0}) || !count(ncw, {C, conv ? p.conv_kernel : 0}) ||
        !count(nal, {HV}) || !count(ndt, {HV, K}))
        return fail(KDA_EINVAL, "kda_decode_step: tensor sizes overflow");
    if (B == 0) return KDA_OK;
    if (!qkv || !gate || !beta || !state || !out)
        return fail(KDA_EINVAL, "kda_decode_step: qkv, gate, beta, state and out must be non-NULL");
    const void *ptrs[] = {qkv, gate, beta, state, out, p.conv_weight, p.conv_state, p.A_log, p.dt_bias};
    const char *names[] = {"qkv", "gate", "beta", "state", "out", "conv_weight", "conv_state", "A_log", "dt_bias"};
    for (int i = 0; i < 9; ++i)
        if (ptrs[i] && !aligned16(ptrs[i]))
            return fail(KDA_EINVAL, "kda_decode_step: %s is not 16-byte aligned", names[i]);
    const bool gp = p.gate_mode != KDA_GATE_DIRECT;
    const Range rs[] = {rng("qkv", qkv, nx * esz), rng("gate", gate, ng * 4), rng("beta", beta, nb * 4),
                        rng("state", state, ns * 4), rng("out", out, no * esz),
                        rng("conv_weight", p.conv_weight, conv ? ncw * 4 : 0),
                        rng("conv_state", conv ? p.conv_state : nullptr, ncs * 4),
                        rng("A_log", gp ? p.A_log : nullptr, nal * 4),
                        rng("dt_bias", gp ? p.dt_bias : nullptr, ndt * 4)};
    // outputs (state, out, conv_state) may not overlap anything else
    const int outs[] = {3, 4, 6};
    for (int o : outs)
        for (int i = 0; i < 9; ++i)
            if (i != o && overlap(rs[o], rs[i]))
                return fail(KDA_EINVAL, "kda_decode_step: %s overlaps %s", rs[o].name, rs[i].name);

    kda::DecodeArgs a{};
    a.qkv = qkv; a.gate = gate; a.beta = beta; a.state = state; a.out = out;
    a.conv_w = p.conv_weight; a.conv_state = conv ? p.conv_state : nullptr;
    a.conv_kernel = conv ? p.conv_kernel : 0;
    a.conv_ring = conv && p.conv_ring ? 1 : 0; a.conv_pos = a.conv_ring ? p.conv_pos : 0;
    a.l2norm = p.l2norm_qk ? 1 : 0; a.l2_eps = p.l2_eps;
    a.gate_mode = p.gate_mode; a.A_log = p.A_log; a.dt_bias = p.dt_bias;
    a.lower_bound = p.gate_lower_bound; a.beta_is_logit = p.beta_is_logit ? 1 : 0;
    a.B = B; a.H = H; a.HV = HV; a.K = K; a.V = V; a.scale = scale;
    a.bf16 = dtype == KDA_DTYPE_BF16;
    const hipError_t e = kda::launch_decode(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KDA_EHIP, "kda_decode_step: launch failed: %s", hipGetErrorString(e));
    return KDA_OK;
}

}  // extern "C"
