// gdn_api.cpp -- C ABI of libgdn: argument validation, launch planning and
// dispatch to the HIP kernels.  Declarations and conventions: include/gdn.h.
#include "gdn.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gdn_kernels.h"

namespace {

constexpr int STEP_CHUNK = 64;   // token tile of gdn_fwd_step

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, const char* detail = nullptr) {
    if (detail)
        snprintf(g_last_error, sizeof(g_last_error), fmt, detail);
    else
        snprintf(g_last_error, sizeof(g_last_error), "%s", fmt);
    return status;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool head_ok(int d) { return d == 32 || d == 64 || d == 128; }

void defaults(gdn_opts* o) {
    o->in_dtype = GDN_BF16;
    o->out_dtype = GDN_F32;
    o->qk_l2norm = 1;
    o->scale = 1.0f;
    o->eps = 1e-6f;
    o->stream = nullptr;
    o->workspace = nullptr;
    o->workspace_bytes = 0;
    o->gate_logits = 0;
    o->out_gate = nullptr;
}

// Debug switch: with GDN_DEBUG_REVERSE_WORKGROUPS set (and not "0") every
// launch's workgroups take their work items in reverse order of dispatch;
// results must not change (checked by the GPU tests).
int debug_reverse_workgroups() {
    const char* e = getenv("GDN_DEBUG_REVERSE_WORKGROUPS");
    return (e && e[0] && !(e[0] == '0' && e[1] == '\0')) ? 1 : 0;
}

// Sizes the calls accept: the limits validate() enforces on B, H and T.
bool sizes_ok(int B, int H, int T, int dk, int dv) {
    return B > 0 && H > 0 && T >= 0 && (long long)B * H * 8 <= 0x7fffffffLL &&
           (long long)T * (dk > dv ? dk : dv) * 4 <= 0x7fffffffLL;
}

int validate(const void* q, const void* k, const void* v, const void* alpha, const void* beta,
             const float* state_in, const void* out, const float* state_out,
             int B, int H, int T, int dk, int dv, int chunk, const gdn_opts& o) {
    if (B <= 0 || H <= 0) return fail(GDN_ERR_ARG, "B and H must be positive");
    if (T < 0) return fail(GDN_ERR_ARG, "T must be non-negative");
    if ((long long)B * H * 8 > 0x7fffffffLL) return fail(GDN_ERR_ARG, "B*H too large");
    if ((long long)T * (dk > dv ? dk : dv) * 4 > 0x7fffffffLL)   // byte ranges of one head below 2 GiB
        return fail(GDN_ERR_ARG, "T too large");
    if (!head_ok(dk)) return fail(GDN_ERR_UNSUPPORTED, "dk must be 32, 64 or 128");
    if (!head_ok(dv)) return fail(GDN_ERR_UNSUPPORTED, "dv must be 32, 64 or 128");
    if (chunk != 32 && chunk != 64 && chunk != 128)
        return fail(GDN_ERR_UNSUPPORTED, "chunk must be 32, 64 or 128");
    if (o.in_dtype != GDN_BF16 && o.in_dtype != GDN_F32) return fail(GDN_ERR_ARG, "bad in_dtype");
    if (o.out_dtype != GDN_BF16 && o.out_dtype != GDN_F32) return fail(GDN_ERR_ARG, "bad out_dtype");
    if (T > 0) {
        if (!q || !k || !v || !alpha || !beta || !out)
            return fail(GDN_ERR_ARG, "q, k, v, alpha, beta and out must be non-null when T > 0");
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
            return fail(GDN_ERR_ARG, "q, k, v and out must be 16-byte aligned");
        if (o.out_gate && !aligned16(o.out_gate))
            return fail(GDN_ERR_ARG, "out_gate must be 16-byte aligned");
        const size_t esz = o.in_dtype == GDN_F32 ? 4 : 2;
        if ((reinterpret_cast<uintptr_t>(alpha) % esz) || (reinterpret_cast<uintptr_t>(beta) % esz))
            return fail(GDN_ERR_ARG, "alpha and beta must be aligned to their element size");
    }
    if (state_in && !aligned16(state_in)) return fail(GDN_ERR_ARG, "state_in must be 16-byte aligned");
    if (state_out && !aligned16(state_out)) return fail(GDN_ERR_ARG, "state_out must be 16-byte aligned");
    return GDN_OK;
}

// Launch plan of one call.
struct Plan {
    bool single;     // single-pass kernel (128-token chunks, or walker does not fit)
    bool pipe;       // pipelined walker (bf16 inputs)
    int bv;          // value-column tile (single) ...
    int waves;       // ... or waves per workgroup of the segmented walker (tile = 16 * waves)
    int nseg;        // sequence segments (walker)
    int seg_chunks;  // chunks per segment
    size_t ws_bytes; // workspace needed for nseg > 1
};

// Single-pass kernel: the widest tile that still gives every compute unit a
// workgroup; below that the narrowest tile (most workgroups).
int single_bv(int in_f32, int B, int H, int dk, int dv, int chunk) {
    const int maxbv = gdn::single_max_bv(in_f32, dk, chunk);
    const long long bh = (long long)B * H;
    const int cand[3] = {64, 32, 16};
    for (int c : cand) {
        if (c > maxbv || dv % c) continue;
        if (bh * (dv / c) >= 256) return c;
    }
    return maxbv < 16 ? maxbv : 16;
}

// Walker plan.  Without segments a sequence is one chain of chunks per
// workgroup; with few heads that leaves most of the 256 compute units idle,
// so the sequence is cut into segments until about one workgroup per compute
// unit is busy (each segment keeps at least two chunks).
size_t seg_workspace(int in_f32, int B, int H, int dk, int dv, int nseg) {
    if (nseg <= 1) return 0;
    const size_t bh = (size_t)B * H, ns = (size_t)(nseg - 1);
    return bh * ns * dk * dk * (in_f32 ? 4 : 2)     // A_s
         + bh * ns * dk * dv * 4                      // B_s
         + bh * dk * dv * 4;                          // snapshot of state_in
}

// Pipelined walker: pick the segment count with the shortest estimated
// critical path, in units of one chunk step of the unsegmented walk.
// Unsegmented, a walk of L chunks takes about L + 1 steps.  Segmented, every
// segment is walked once on [identity | value] columns (heavier steps), then
// the correction pass pays a launch and its first memory round trips, one
// folded map per preceding segment and the rewrite of the segment's outputs.
// A launch of more workgroups than compute units runs in rounds.  Constants
// measured on MI355X.  walks = 2: a fused bidirectional call, whose launches
// walk and correct both directions at once.  plain: no gates, not reversed,
// not accumulating; segment 0 then walks from state_in and needs no
// correction (one folded map fewer), and the pass starts sooner and rewrites
// a chunk faster, since it loads no gate or accumulation operands (refitted
// to the 16-head rollout, streaming chunk and 48-head single-frame step).
Plan pipe_plan(int B, int H, int T, int dk, int dv, int chunk, int walks = 1, bool plain = false) {
    Plan pl{};
    pl.pipe = true;
    const int nchunks = (int)(((long long)T + chunk - 1) / chunk);
    const long long bh = (long long)B * H;
    const long long base = bh * (dv / 64);                                  // workgroups, unsegmented
    const int cts = gdn::pipe_seg_tiles(dk, dv);
    const long long sb = walks * bh * ((dk + dv) / (64 * cts));             // per segment
    const double step_us = (dk == 64 ? 2.7 : 4.0) * (chunk == 64 ? 1.0 : 0.6);
    const double wstep = dk == 64 ? 1.45 : 1.33;         // segment-walk step / unsegmented step
    const double fix = (plain ? 5.0 : 9.0) / step_us;    // correction pass: launch, first loads
    const double fold = 0.15;                             // one folded map
    const double corr = (plain ? 0.2 : 0.3) * chunk / 64; // outputs of one chunk rewritten
    auto rounds = [](long long wgs) { return (double)((wgs + 255) / 256); };
    int best_n = 0;
    double best = 0;
    for (int n = 2; n <= 64 && 2 * n <= nchunks; ++n) {
        const int L = (nchunks + n - 1) / n;
        const int ns = (nchunks + L - 1) / L;
        if (ns < 2 || ns != n) continue;
        const int nfold = plain ? ns - 2 : ns - 1;       // maps folded by the last segment
        // the correction pass runs in rounds too (one workgroup per head, 64
        // value columns and corrected segment): five segments of the 48-head
        // single-frame step, two rounds of each launch, measured 61 us per
        // call against 51 us for two segments in one round
        const long long fixw = bh * (dv / 64) * (plain ? ns - 1 : ns);
        const double cost = rounds(sb * ns) * (L + 1) * wstep + rounds(fixw) * (fix + fold * nfold + corr * walks * L);
        if (best_n == 0 || cost < best) { best = cost; best_n = ns; }
    }
    // segments only for a clear gain over the unsegmented walk
    if (best_n == 0 || best > 0.9 * rounds(base) * (nchunks + 1)) best_n = 1;
    pl.nseg = best_n;
    pl.seg_chunks = best_n > 1 ? (nchunks + best_n - 1) / best_n : (nchunks > 0 ? nchunks : 1);
    pl.ws_bytes = gdn::pipe_workspace(B, H, dk, dv, chunk, pl.nseg, pl.seg_chunks);
    return pl;
}

Plan make_plan(int in_f32, int B, int H, int T, int dk, int dv, int chunk, bool plain) {
    if (gdn::pipe_supported(in_f32, dk, dv, chunk)) return pipe_plan(B, H, T, dk, dv, chunk, 1, plain);
    Plan pl{};
    int w = chunk == 128 ? 0 : gdn::walk_max_waves(in_f32, dk, chunk);
    while (w > 0 && (16 * w > dk || 16 * w > dv)) w >>= 1;
    if (w < 2) w = 0;
    if (w == 0) {
        pl.single = true;
        pl.bv = single_bv(in_f32, B, H, dk, dv, chunk);
        pl.nseg = 1;
        return pl;
    }
    pl.waves = w;
    const int nchunks = (int)(((long long)T + chunk - 1) / chunk);
    const long long base = (long long)B * H * (w ? dv / (16 * w) : 1);
    int nseg = 1;
    if (nchunks >= 4 && base < 256) {
        const long long want = (256 + base - 1) / base;
        int L = (int)((nchunks + want - 1) / want);
        if (L < 2) L = 2;
        nseg = (nchunks + L - 1) / L;
    }
    pl.nseg = nseg < 1 ? 1 : nseg;
    pl.seg_chunks = (nchunks + pl.nseg - 1) / pl.nseg;
    if (pl.seg_chunks < 1) pl.seg_chunks = 1;
    pl.nseg = nchunks > 0 ? (nchunks + pl.seg_chunks - 1) / pl.seg_chunks : 1;
    pl.ws_bytes = seg_workspace(in_f32, B, H, dk, dv, pl.nseg);
    return pl;
}

// Segment data of the pipelined walker at w (gdn::pipe_workspace bytes): the
// maps of all nseg segments, the copy of state_in, Phi, the partial outputs
// and the working scales.
void carve_pipe(char* w, size_t bh, int nseg, int seg_chunks, int chunk, int dk, int dv, void** summA,
                float** summB, float** snap, void** phi, void** ostage, float** sscale) {
    const size_t ns = (size_t)nseg, rows = (size_t)seg_chunks * chunk;
    *summA = w;
    *summB = reinterpret_cast<float*>(w + bh * ns * dk * dk * 2);
    *snap = *summB + bh * ns * dk * dv;
    char* ph = reinterpret_cast<char*>(*snap + bh * dk * dv);
    *phi = ph;
    *ostage = ph + bh * ns * rows * dk * 2;
    *sscale = reinterpret_cast<float*>(reinterpret_cast<char*>(*ostage) + bh * ns * rows * dv * 2);
}

// One scan over the sequence.  reverse: walk the tokens backward; accumulate:
// add the outputs to out (fp32 out), or add acc_src before rounding (bf16
// out).  Arguments are validated by the caller.
int scan(const void* q, const void* k, const void* v, const void* alpha, const void* beta,
         const float* state_in, void* out, float* state_out,
         int B, int H, int T, int dk, int dv, int chunk, const gdn_opts& o, int reverse, int accumulate,
         const float* acc_src = nullptr) {
    gdn::WalkArgs a{};
    a.rev_wg = debug_reverse_workgroups();
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta;
    a.state_in = state_in; a.out = out; a.state_out = state_out;
    a.B = B; a.H = H; a.T = T; a.dk = dk; a.dv = dv;
    a.scale = o.scale; a.eps = o.eps; a.qk_l2norm = o.qk_l2norm ? 1 : 0;
    a.out_bf16 = o.out_dtype == GDN_BF16; a.in_f32 = o.in_dtype == GDN_F32;
    a.gate_logits = o.gate_logits ? 1 : 0;
    a.out_gate = o.out_gate;
    a.reverse = reverse;
    a.accumulate = accumulate;
    a.acc_src = acc_src;
    if (T == 0 && !state_out) return GDN_OK;
    // the same test as the launch's choice of the plain walker (no gates, not
    // reversed, not accumulating)
    const bool plain = !a.gate_logits && !a.out_gate && !reverse && !accumulate;
    Plan pl = make_plan(a.in_f32, B, H, T, dk, dv, chunk, plain);
    hipStream_t stream = reinterpret_cast<hipStream_t>(o.stream);
    hipError_t e;
    if (pl.single) {
        if (pl.bv == 0)
            return fail(GDN_ERR_UNSUPPORTED, "this chunk does not fit on chip for fp32 inputs at this dk");
        e = gdn::launch_fwd_single(a, chunk, pl.bv, stream);
    } else {
        if (pl.nseg > 1 && (!o.workspace || o.workspace_bytes < pl.ws_bytes)) {
            pl.nseg = 1;                       // no workspace: unsplit walk
            pl.seg_chunks = (int)(((long long)T + chunk - 1) / chunk);
        }
        if (pl.seg_chunks < 1) pl.seg_chunks = 1;
        a.nseg = pl.nseg;
        a.seg_chunks = pl.seg_chunks;
        a.summA = nullptr; a.summB = nullptr; a.snap = nullptr; a.phi = nullptr; a.ostage = nullptr;
        a.sscale = nullptr;
        if (pl.nseg > 1) {
            const size_t bh = (size_t)B * H;
            char* w = reinterpret_cast<char*>(o.workspace);
            if (pl.pipe) {
                carve_pipe(w, bh, pl.nseg, pl.seg_chunks, chunk, dk, dv, &a.summA, &a.summB, &a.snap, &a.phi,
                           &a.ostage, &a.sscale);
            } else {
                // maps of segments 0 .. nseg-2
                const size_t ns = (size_t)(pl.nseg - 1);
                a.summA = w;
                a.summB = reinterpret_cast<float*>(w + bh * ns * dk * dk * (a.in_f32 ? 4 : 2));
                a.snap = a.summB + bh * ns * dk * dv;
            }
        }
        if (pl.nseg > 1 && (reinterpret_cast<uintptr_t>(o.workspace) & 15u))
            return fail(GDN_ERR_ARG, "workspace must be 16-byte aligned");
        e = pl.pipe ? gdn::launch_pipe(a, chunk, stream) : gdn::launch_walk(a, chunk, pl.waves, stream);
    }
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return GDN_OK;
}

int run(const void* q, const void* k, const void* v, const void* alpha, const void* beta,
        const float* state_in, void* out, float* state_out,
        int B, int H, int T, int dk, int dv, int chunk, const gdn_opts* opts) {
    g_last_error[0] = '\0';
    gdn_opts o;
    if (opts) o = *opts; else defaults(&o);
    int st = validate(q, k, v, alpha, beta, state_in, out, state_out, B, H, T, dk, dv, chunk, o);
    if (st != GDN_OK) return st;
    return scan(q, k, v, alpha, beta, state_in, out, state_out, B, H, T, dk, dv, chunk, o, 0, 0);
}

// The fp32 plane of a bidirectional call (the backward scan's outputs) at the
// start of its workspace, 256-byte aligned; the segment data follow it.
size_t plane_bytes(int B, int H, int T, int dv) {
    return ((size_t)B * H * T * dv * 4 + 255) & ~(size_t)255;
}
size_t bidir_workspace(int B, int H, int T, int dk, int dv, int chunk, const gdn_opts& o);

// Fused bidirectional plan: the pipelined walker with segments, both
// directions walked by one launch and corrected by one pass that writes the
// sum (no plane).  The segment count is planned for the doubled launch; the
// workspace holds one set of segment data per direction.  nseg <= 1: the
// fused path does not apply.
Plan bidir_fused_plan(const gdn_opts& o, int B, int H, int T, int dk, int dv, int chunk) {
    Plan pl{};
    if (!gdn::pipe_supported(o.in_dtype == GDN_F32, dk, dv, chunk)) return pl;
    pl = pipe_plan(B, H, T, dk, dv, chunk, 2, false);
    if (pl.nseg > 1) pl.ws_bytes = 2 * ((pl.ws_bytes + 255) & ~(size_t)255);
    return pl;
}

int scan_bidir_fused(const void* q, const void* k, const void* v, const void* alpha, const void* beta,
                     const float* state_in, void* out, float* state_out,
                     int B, int H, int T, int dk, int dv, int chunk, const gdn_opts& o, const Plan& pl) {
    gdn::WalkArgs a{};
    a.rev_wg = debug_reverse_workgroups();
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta;
    a.state_in = state_in; a.out = out; a.state_out = state_out;
    a.B = B; a.H = H; a.T = T; a.dk = dk; a.dv = dv;
    a.scale = o.scale; a.eps = o.eps; a.qk_l2norm = o.qk_l2norm ? 1 : 0;
    a.out_bf16 = o.out_dtype == GDN_BF16; a.in_f32 = 0;
    a.gate_logits = o.gate_logits ? 1 : 0;
    a.out_gate = o.out_gate;
    a.bidir = 1;
    a.nseg = pl.nseg;
    a.seg_chunks = pl.seg_chunks;
    const size_t bh = (size_t)B * H;
    char* w = reinterpret_cast<char*>(o.workspace);
    carve_pipe(w, bh, pl.nseg, pl.seg_chunks, chunk, dk, dv, &a.summA, &a.summB, &a.snap, &a.phi, &a.ostage,
               &a.sscale);
    float* unused_snap = nullptr;
    carve_pipe(w + pl.ws_bytes / 2, bh, pl.nseg, pl.seg_chunks, chunk, dk, dv, &a.bw.summA, &a.bw.summB,
               &unused_snap, &a.bw.phi, &a.bw.ostage, &a.bw.sscale);
    hipError_t e = gdn::launch_pipe(a, chunk, reinterpret_cast<hipStream_t>(o.stream));
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return GDN_OK;
}

// Bidirectional.  Fused (pipelined walker with segments, and a workspace of
// gdn_bidir_workspace_bytes): one launch walks both directions' segments, one
// correction pass writes the sum.  Otherwise: the backward scan (zero state,
// tokens in reverse, no state kept) writes its fp32 outputs to the plane,
// then the forward scan from state_in adds the plane to its own outputs
// before their one rounding and writes state_out.  The output gate is applied
// in both (it distributes over the sum).  Stream order keeps the two scans
// apart, so they share the segment data; a workspace of the plane alone runs
// both scans unsplit.
int run_bidir(const void* q, const void* k, const void* v, const void* alpha, const void* beta,
              const float* state_in, void* out, float* state_out,
              int B, int H, int T, int dk, int dv, int chunk, const gdn_opts* opts) {
    g_last_error[0] = '\0';
    gdn_opts o;
    if (opts) o = *opts; else defaults(&o);
    int st = validate(q, k, v, alpha, beta, state_in, out, state_out, B, H, T, dk, dv, chunk, o);
    if (st != GDN_OK) return st;
    if (T == 0) return scan(q, k, v, alpha, beta, state_in, out, state_out, B, H, T, dk, dv, chunk, o, 0, 0);
    const size_t pb = plane_bytes(B, H, T, dv);
    if (!o.workspace || o.workspace_bytes < pb || !aligned16(o.workspace)) {
        char n[32];
        snprintf(n, sizeof(n), "%zu", bidir_workspace(B, H, T, dk, dv, chunk, o));
        return fail(GDN_ERR_ARG, "gdn_fwd_bidir needs a 16-byte aligned workspace of at least the "
                    "fp32 plane (gdn_bidir_workspace_bytes() = %s bytes with the segment data)", n);
    }
    const Plan fp = bidir_fused_plan(o, B, H, T, dk, dv, chunk);
    if (fp.nseg > 1 && o.workspace_bytes >= fp.ws_bytes)
        return scan_bidir_fused(q, k, v, alpha, beta, state_in, out, state_out, B, H, T, dk, dv, chunk, o, fp);
    float* plane = reinterpret_cast<float*>(o.workspace);
    gdn_opts os = o;                               // segment data after the plane
    os.workspace = reinterpret_cast<char*>(o.workspace) + pb;
    os.workspace_bytes = o.workspace_bytes - pb;
    gdn_opts ob = os;
    ob.out_dtype = GDN_F32;
    st = scan(q, k, v, alpha, beta, nullptr, plane, nullptr, B, H, T, dk, dv, chunk, ob, 1, 0);
    if (st != GDN_OK) return st;
    return scan(q, k, v, alpha, beta, state_in, out, state_out, B, H, T, dk, dv, chunk, os, 0, 1, plane);
}

size_t workspace_for(int B, int H, int T, int dk, int dv, int chunk, const gdn_opts* opts) {
    gdn_opts o;
    if (opts) o = *opts; else defaults(&o);
    if (!sizes_ok(B, H, T, dk, dv) || !head_ok(dk) || !head_ok(dv)) return 0;
    if (chunk != 32 && chunk != 64 && chunk != 128) return 0;
    // a forward call's plan (plain without gates), as the call itself makes it
    Plan pl = make_plan(o.in_dtype == GDN_F32, B, H, T, dk, dv, chunk, !o.gate_logits && !o.out_gate);
    return pl.ws_bytes;
}

size_t bidir_workspace(int B, int H, int T, int dk, int dv, int chunk, const gdn_opts& o) {
    if (!sizes_ok(B, H, T, dk, dv) || !head_ok(dk) || !head_ok(dv)) return 0;
    if (chunk != 32 && chunk != 64 && chunk != 128) return 0;
    if (T == 0) return 0;
    const size_t pb = plane_bytes(B, H, T, dv);
    const Plan fp = bidir_fused_plan(o, B, H, T, dk, dv, chunk);
    if (fp.nseg > 1) return fp.ws_bytes > pb ? fp.ws_bytes : pb;
    // the two scans reverse or accumulate: not plain
    const Plan pl = make_plan(o.in_dtype == GDN_F32, B, H, T, dk, dv, chunk, false);
    return pb + pl.ws_bytes;
}

// Frame-wise Gated DeltaNet with a normalised readout: frame summaries, a
// scan over frames, the readout (gdn_frame.hip).  The workspace holds the
// summaries of every (head, frame, token split), each frame's state in the
// form the readout reads, and z_f.
bool frame_shape_ok(int B, int H, int F, int N, int dk, int dv) {
    return B > 0 && H > 0 && F >= 0 && N > 0 && (dk == 64 || dk == 128) && (dv == 64 || dv == 128) &&
           (long long)B * H <= 65535 && F <= 65535;
}

int run_framewise(const void* q, const void* k, const void* v, const void* alpha, const void* beta,
                  const float* state_in, const float* z_in, void* out, float* state_out, float* z_out,
                  int B, int H, int F, int N, int dk, int dv, const gdn_opts* opts) {
    g_last_error[0] = '\0';
    gdn_opts o;
    if (opts) o = *opts; else defaults(&o);
    if (B <= 0 || H <= 0 || F < 0 || N <= 0) return fail(GDN_ERR_ARG, "B, H and N must be positive, F non-negative");
    if (o.in_dtype != GDN_BF16) return fail(GDN_ERR_UNSUPPORTED, "frame-wise inputs must be bf16");
    if (o.out_dtype != GDN_BF16 && o.out_dtype != GDN_F32) return fail(GDN_ERR_ARG, "bad out_dtype");
    if (!frame_shape_ok(B, H, F, N, dk, dv))
        return fail(GDN_ERR_UNSUPPORTED, "frame-wise: dk and dv 64 or 128, B*H and F at most 65535");
    if ((long long)F * N > 0x7fffffffLL) return fail(GDN_ERR_ARG, "F*N too large");
    if (F > 0) {
        if (!q || !k || !v || !alpha || !beta || !out)
            return fail(GDN_ERR_ARG, "q, k, v, alpha, beta and out must be non-null when F > 0");
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
            return fail(GDN_ERR_ARG, "q, k, v and out must be 16-byte aligned");
        if (o.out_gate && !aligned16(o.out_gate)) return fail(GDN_ERR_ARG, "out_gate must be 16-byte aligned");
        if ((reinterpret_cast<uintptr_t>(alpha) & 1u) || (reinterpret_cast<uintptr_t>(beta) & 1u))
            return fail(GDN_ERR_ARG, "alpha and beta must be aligned to their element size");
    }
    if ((state_in && !aligned16(state_in)) || (state_out && !aligned16(state_out)) ||
        (z_in && !aligned16(z_in)) || (z_out && !aligned16(z_out)))
        return fail(GDN_ERR_ARG, "states must be 16-byte aligned");
    size_t off_mt = 0, off_zf = 0;
    const size_t need = F > 0 ? gdn::frame_workspace(B, H, F, N, dk, dv, &off_mt, &off_zf) : 0;
    if (need > 0 && (!o.workspace || o.workspace_bytes < need || !aligned16(o.workspace))) {
        char n[32];
        snprintf(n, sizeof(n), "%zu", need);
        return fail(GDN_ERR_ARG, "gdn_fwd_framewise needs a 16-byte aligned workspace of "
                    "gdn_framewise_workspace_bytes() = %s bytes", n);
    }
    if (F == 0 && !state_out && !z_out) return GDN_OK;
    gdn::FrameArgs a{};
    a.rev_wg = debug_reverse_workgroups();
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta;
    a.state_in = state_in; a.z_in = z_in; a.out = out; a.state_out = state_out; a.z_out = z_out;
    a.out_gate = o.out_gate;
    a.B = B; a.H = H; a.F = F; a.N = N; a.dk = dk; a.dv = dv;
    a.gate_logits = o.gate_logits ? 1 : 0;
    a.qk_l2norm = o.qk_l2norm ? 1 : 0;
    a.out_bf16 = o.out_dtype == GDN_BF16;
    a.eps = o.eps;
    gdn::frame_plan(B, H, F, N, dk, dv, &a.nsp, &a.nts);
    if ((long long)(dv / 64) * a.nts * F * B * H > 0x7fffffffLL)
        return fail(GDN_ERR_UNSUPPORTED, "frame-wise: too many readout workgroups (B*H*F too large)");
    char* w = reinterpret_cast<char*>(o.workspace);
    a.sums = reinterpret_cast<float*>(w);
    a.mt_hi = reinterpret_cast<uint16_t*>(w + off_mt);
    a.mt_lo = reinterpret_cast<uint16_t*>(w + off_mt + (off_zf - off_mt) / 2);
    a.zf = reinterpret_cast<float*>(w + off_zf);
    hipError_t e = gdn::launch_framewise(a, reinterpret_cast<hipStream_t>(o.stream));
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return GDN_OK;
}

}  // namespace

int gdn::api_fail(int status, const char* msg) { return fail(status, "%s", msg); }

extern "C" {

void gdn_default_opts(gdn_opts* opts) {
    if (opts) defaults(opts);
}

int gdn_fwd_chunked(const void* q, const void* k, const void* v, const void* alpha, const void* beta,
                    const float* state_in, void* out, float* state_out,
                    int B, int H, int T, int dk, int dv, int chunk, const gdn_opts* opts) {
    return run(q, k, v, alpha, beta, state_in, out, state_out, B, H, T, dk, dv, chunk, opts);
}

int gdn_fwd_step(const void* q, const void* k, const void* v, const void* alpha, const void* beta,
                 const float* state_in, void* out, float* state_out,
                 int B, int H, int T, int dk, int dv, const gdn_opts* opts) {
    return run(q, k, v, alpha, beta, state_in, out, state_out, B, H, T, dk, dv, STEP_CHUNK, opts);
}

int gdn_fwd_bidir(const void* q, const void* k, const void* v, const void* alpha, const void* beta,
                  const float* state_in, void* out, float* state_out,
                  int B, int H, int T, int dk, int dv, int chunk, const gdn_opts* opts) {
    return run_bidir(q, k, v, alpha, beta, state_in, out, state_out, B, H, T, dk, dv,
                     chunk > 0 ? chunk : STEP_CHUNK, opts);
}

int gdn_attn_sink_window(const void* q, const void* k_sink, const void* v_sink, int n_sink,
                         const void* k_win, const void* v_win, int n_win,
                         const void* k_cur, const void* v_cur, int n_cur,
                         void* out, int B, int H, int Nq, int d, float scale, const gdn_opts* opts) {
    g_last_error[0] = '\0';
    gdn_opts o;
    if (opts) o = *opts; else defaults(&o);
    if (B < 0 || H < 0 || Nq < 0 || n_sink < 0 || n_win < 0 || n_cur < 0)
        return fail(GDN_ERR_ARG, "negative size");
    if (!gdn::attn_supported(d)) return fail(GDN_ERR_UNSUPPORTED, "d must be 64 or 128");
    if (o.in_dtype != GDN_BF16) return fail(GDN_ERR_UNSUPPORTED, "attention inputs must be bf16");
    if (o.out_dtype != GDN_BF16 && o.out_dtype != GDN_F32) return fail(GDN_ERR_ARG, "bad out_dtype");
    if ((long long)B * H * Nq == 0) return GDN_OK;
    if (n_sink + n_win + n_cur <= 0) return fail(GDN_ERR_ARG, "empty key set");
    const long long lim = 0x7fffffffLL;
    if ((long long)Nq * d * 4 > lim || (long long)n_sink * d * 2 > lim || (long long)n_win * d * 2 > lim ||
        (long long)n_cur * d * 2 > lim)
        return fail(GDN_ERR_UNSUPPORTED, "per-head size above 2 GiB");
    if (!q || !out) return fail(GDN_ERR_ARG, "q and out must not be NULL");
    const void* ks[3] = {k_sink, k_win, k_cur};
    const void* vs[3] = {v_sink, v_win, v_cur};
    const int ns[3] = {n_sink, n_win, n_cur};
    for (int i = 0; i < 3; ++i) {
        if (ns[i] > 0 && (!ks[i] || !vs[i])) return fail(GDN_ERR_ARG, "keys and values of a non-empty segment must not be NULL");
        if (ns[i] > 0 && (!aligned16(ks[i]) || !aligned16(vs[i]))) return fail(GDN_ERR_ARG, "keys and values must be 16-byte aligned");
    }
    if (!aligned16(q) || !aligned16(out)) return fail(GDN_ERR_ARG, "q and out must be 16-byte aligned");
    gdn::AttnArgs a{};
    a.rev_wg = debug_reverse_workgroups();
    a.q = q;
    for (int i = 0; i < 3; ++i) {
        a.k[i] = ks[i];
        a.v[i] = vs[i];
        a.n[i] = ns[i];
    }
    a.out = out;
    a.B = B; a.H = H; a.Nq = Nq; a.d = d;
    a.scale = scale > 0.f ? scale : 1.f / sqrtf((float)d);
    a.out_bf16 = o.out_dtype == GDN_BF16;
    // key ranges split over workgroups when the caller's workspace holds them
    a.nsplit = gdn::attn_splits(B, H, Nq, ns);
    a.part_o = nullptr;
    a.part_ml = nullptr;
    const size_t need = gdn::attn_workspace(B, H, Nq, d, a.nsplit);
    if (a.nsplit > 1 && (!o.workspace || o.workspace_bytes < need || !aligned16(o.workspace))) a.nsplit = 1;
    if (a.nsplit > 1) {
        a.part_o = reinterpret_cast<float*>(o.workspace);
        a.part_ml = a.part_o + (size_t)a.nsplit * B * H * Nq * d;
    }
    hipError_t e = gdn::launch_attn(a, reinterpret_cast<hipStream_t>(o.stream));
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return GDN_OK;
}

size_t gdn_attn_workspace_bytes(int B, int H, int Nq, int n_sink, int n_win, int n_cur, int d,
                                const gdn_opts* opts) {
    (void)opts;
    if (B <= 0 || H <= 0 || Nq <= 0 || n_sink < 0 || n_win < 0 || n_cur < 0 || !gdn::attn_supported(d)) return 0;
    const int ns[3] = {n_sink, n_win, n_cur};
    return gdn::attn_workspace(B, H, Nq, d, gdn::attn_splits(B, H, Nq, ns));
}

size_t gdn_bidir_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, const gdn_opts* opts) {
    gdn_opts o;
    if (opts) o = *opts; else defaults(&o);
    return bidir_workspace(B, H, T, dk, dv, chunk > 0 ? chunk : STEP_CHUNK, o);
}

size_t gdn_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, const gdn_opts* opts) {
    return workspace_for(B, H, T, dk, dv, chunk > 0 ? chunk : STEP_CHUNK, opts);
}

int gdn_fwd_framewise(const void* q, const void* k, const void* v, const void* alpha, const void* beta,
                      const float* state_in, const float* z_in, void* out, float* state_out, float* z_out,
                      int B, int H, int F, int N, int dk, int dv, int chunk, const gdn_opts* opts) {
    (void)chunk;
    return run_framewise(q, k, v, alpha, beta, state_in, z_in, out, state_out, z_out, B, H, F, N, dk, dv, opts);
}

size_t gdn_framewise_workspace_bytes(int B, int H, int F, int N, int dk, int dv, int chunk,
                                     const gdn_opts* opts) {
    (void)opts;
    (void)chunk;
    if (!frame_shape_ok(B, H, F, N, dk, dv) || F == 0) return 0;
    return gdn::frame_workspace(B, H, F, N, dk, dv, nullptr, nullptr);
}

const char* gdn_strerror(int status) {
    switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_ARG: return "invalid argument";
    case GDN_ERR_UNSUPPORTED: return "unsupported shape or option";
    case GDN_ERR_HIP: return "HIP error";
    default: return "unknown status";
    }
}

const char* gdn_last_error(void) { return g_last_error; }

int gdn_version(void) { return GDN_VERSION; }

int gdn_debug_flags(void) { return debug_reverse_workgroups(); }

}  // extern "C"
