// Host-side checks of libgdn's C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer: argument validation, workspace sizing and the
// error text, all of which return before any HIP call, so this runs without a
// GPU.  Built by tests/test_sanitize.py with the API source compiled by the
// host compiler (sanitized) and the kernels' host objects linked as built.
// Prints one line per failed expectation and exits non-zero if any failed.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gdn.h"

static int g_fail = 0;

#define EXPECT(cond, ...)                                            \
    do {                                                             \
        if (!(cond)) {                                               \
            ++g_fail;                                                \
            printf("FAIL line %d: ", __LINE__);                      \
            printf(__VA_ARGS__);                                     \
            printf(" [last error: %s]\n", gdn_last_error());         \
        }                                                            \
    } while (0)

// Fake device addresses: validation reads pointer values only.
static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }
static const uintptr_t A = 0x10000;          // 16-byte aligned

static int chunked(int B, int H, int T, int dk, int dv, int chunk, const gdn_opts* o,
                   uintptr_t q = A, uintptr_t out = A) {
    return gdn_fwd_chunked(P(q), P(A), P(A), P(A), P(A), nullptr, P(out), nullptr,
                           B, H, T, dk, dv, chunk, o);
}

int main() {
    EXPECT(gdn_version() == GDN_VERSION, "version %d", gdn_version());
    const int codes[] = {0, -1, -2, -3, 7, -100};
    for (int s : codes) EXPECT(gdn_strerror(s) && gdn_strerror(s)[0], "strerror(%d)", s);
    gdn_default_opts(nullptr);
    gdn_opts o;
    memset(&o, 0x5a, sizeof(o));
    gdn_default_opts(&o);
    EXPECT(o.in_dtype == GDN_BF16 && o.out_dtype == GDN_F32 && o.qk_l2norm == 1 && o.scale == 1.f &&
               o.workspace == nullptr && o.workspace_bytes == 0 && o.stream == nullptr &&
               o.gate_logits == 0 && o.out_gate == nullptr,
           "defaults");

    // ---- gdn_fwd_chunked / gdn_fwd_step argument errors
    EXPECT(chunked(1, 2, 100, 64, 64, 16, nullptr) == GDN_ERR_UNSUPPORTED, "chunk 16");
    EXPECT(strlen(gdn_last_error()) > 0, "error text after a refusal");
    EXPECT(chunked(1, 2, 100, 64, 64, 48, nullptr) == GDN_ERR_UNSUPPORTED, "chunk 48");
    EXPECT(chunked(1, 2, 100, 48, 64, 64, nullptr) == GDN_ERR_UNSUPPORTED, "dk 48");
    EXPECT(chunked(1, 2, 100, 64, 256, 64, nullptr) == GDN_ERR_UNSUPPORTED, "dv 256");
    EXPECT(chunked(-1, 2, 100, 64, 64, 64, nullptr) == GDN_ERR_ARG, "B < 0");
    EXPECT(chunked(1, -2, 100, 64, 64, 64, nullptr) == GDN_ERR_ARG, "H < 0");
    EXPECT(chunked(1, 2, -5, 64, 64, 64, nullptr) == GDN_ERR_ARG, "T < 0");
    EXPECT(chunked(1, 2, 100, 64, 64, 64, nullptr, 0) == GDN_ERR_ARG, "q NULL");
    EXPECT(chunked(1, 2, 100, 64, 64, 64, nullptr, A, 0) == GDN_ERR_ARG, "out NULL");
    EXPECT(chunked(1, 2, 100, 64, 64, 64, nullptr, A + 8) == GDN_ERR_ARG, "q misaligned");
    EXPECT(chunked(65536, 65536, 1 << 30, 128, 128, 64, nullptr) != GDN_OK, "shape beyond 32-bit indexing");
    EXPECT(chunked(1, 1, 0x7fffffff, 128, 128, 64, nullptr) != GDN_OK, "T at INT_MAX");
    {
        gdn_opts f = o;
        f.in_dtype = GDN_F32;
        EXPECT(chunked(1, 2, 100, 64, 64, 128, &f) == GDN_ERR_UNSUPPORTED, "fp32 with chunk 128");
        f.in_dtype = 5;
        EXPECT(chunked(1, 2, 100, 64, 64, 64, &f) != GDN_OK, "bad in_dtype");
        f = o;
        f.out_dtype = 9;
        EXPECT(chunked(1, 2, 100, 64, 64, 64, &f) != GDN_OK, "bad out_dtype");
        f = o;
        f.out_gate = P(A + 4);
        EXPECT(chunked(1, 2, 100, 64, 64, 64, &f) == GDN_ERR_ARG, "out_gate misaligned");
    }
    EXPECT(gdn_fwd_step(P(A), P(A), P(A), P(A), P(A), nullptr, P(A), nullptr, 1, 2, 100, 64, 33, nullptr) ==
               GDN_ERR_UNSUPPORTED,
           "step dv 33");
    EXPECT(gdn_fwd_step(P(A), P(A), nullptr, P(A), P(A), nullptr, P(A), nullptr, 1, 2, 100, 64, 64, nullptr) ==
               GDN_ERR_ARG,
           "step v NULL");

    // ---- gdn_fwd_step_noalloc: plans above the static scratch are refused
    EXPECT(gdn_workspace_bytes(1, 16, 100000, 128, 128, 0, nullptr) > GDN_NOALLOC_SCRATCH_BYTES,
           "a shape whose plan exceeds the scratch");
    EXPECT(gdn_fwd_step_noalloc(P(A), P(A), P(A), P(A), P(A), nullptr, P(A), nullptr, 1, 16, 100000, 128, 128,
                                nullptr) == GDN_ERR_UNSUPPORTED,
           "noalloc above the scratch");
    EXPECT(gdn_fwd_step_noalloc(P(A), P(A), P(A), P(A), P(A), nullptr, P(A), nullptr, 1, 2, 100, 48, 64,
                                nullptr) == GDN_ERR_UNSUPPORTED,
           "noalloc dk 48");

    // ---- gdn_fwd_bidir: the fp32 plane is required
    EXPECT(gdn_fwd_bidir(P(A), P(A), P(A), P(A), P(A), nullptr, P(A), nullptr, 1, 2, 100, 64, 64, 0, nullptr) ==
               GDN_ERR_ARG,
           "bidir without workspace");
    {
        gdn_opts w = o;
        w.workspace = P(A);
        w.workspace_bytes = (size_t)2 * 100 * 64 * 4 - 16;
        EXPECT(gdn_fwd_bidir(P(A), P(A), P(A), P(A), P(A), nullptr, P(A), nullptr, 1, 2, 100, 64, 64, 0, &w) ==
                   GDN_ERR_ARG,
               "bidir workspace one piece short");
        w.workspace = P(A + 8);
        w.workspace_bytes = 1 << 20;
        EXPECT(gdn_fwd_bidir(P(A), P(A), P(A), P(A), P(A), nullptr, P(A), nullptr, 1, 2, 100, 64, 64, 0, &w) ==
                   GDN_ERR_ARG,
               "bidir workspace misaligned");
    }

    // ---- gdn_fwd_framewise
    {
        gdn_opts f = o;
        f.in_dtype = GDN_F32;
        EXPECT(gdn_fwd_framewise(P(A), P(A), P(A), P(A), P(A), nullptr, nullptr, P(A), nullptr, nullptr, 1, 2, 3,
                                 880, 64, 64, 0, &f) == GDN_ERR_UNSUPPORTED,
               "framewise fp32");
        EXPECT(gdn_fwd_framewise(P(A), P(A), P(A), P(A), P(A), nullptr, nullptr, P(A), nullptr, nullptr, 1, 2, 3,
                                 880, 32, 64, 0, nullptr) == GDN_ERR_UNSUPPORTED,
               "framewise dk 32");
        EXPECT(gdn_fwd_framewise(P(A), P(A), P(A), P(A), P(A), nullptr, nullptr, P(A), nullptr, nullptr, 1, 2, -1,
                                 880, 64, 64, 0, nullptr) == GDN_ERR_ARG,
               "framewise F < 0");
        EXPECT(gdn_fwd_framewise(P(A), P(A), P(A), P(A), P(A), nullptr, nullptr, P(A), nullptr, nullptr, 1, 2, 3,
                                 880, 64, 64, 0, nullptr) == GDN_ERR_ARG,
               "framewise without workspace");
        const size_t need = gdn_framewise_workspace_bytes(1, 2, 3, 880, 64, 64, 0, nullptr);
        EXPECT(need > 0 && need % 16 == 0, "framewise workspace %zu", need);
        EXPECT(gdn_framewise_workspace_bytes(1, 2, 0, 880, 64, 64, 0, nullptr) == 0, "framewise F = 0");
        f = o;
        f.workspace = P(A);
        f.workspace_bytes = need - 16;
        EXPECT(gdn_fwd_framewise(P(A), P(A), P(A), P(A), P(A), nullptr, nullptr, P(A), nullptr, nullptr, 1, 2, 3,
                                 880, 64, 64, 0, &f) == GDN_ERR_ARG,
               "framewise workspace short");
        EXPECT(gdn_fwd_framewise(nullptr, P(A), P(A), P(A), P(A), nullptr, nullptr, P(A), nullptr, nullptr, 1, 2, 3,
                                 880, 64, 64, 0, nullptr) == GDN_ERR_ARG,
               "framewise q NULL");
        EXPECT(gdn_fwd_framewise(P(A), P(A), P(A), P(A + 1), P(A), nullptr, nullptr, P(A), nullptr, nullptr, 1, 2,
                                 3, 880, 64, 64, 0, nullptr) == GDN_ERR_ARG,
               "framewise alpha odd address");
    }

    // ---- gdn_attn_sink_window
    EXPECT(gdn_attn_sink_window(P(A), P(A), P(A), 10, nullptr, nullptr, 0, P(A), P(A), 10, P(A), 1, 2, 10, 32, 0.f,
                                nullptr) == GDN_ERR_UNSUPPORTED,
           "attn d 32");
    EXPECT(gdn_attn_sink_window(P(A), nullptr, nullptr, 0, nullptr, nullptr, 0, nullptr, nullptr, 0, P(A), 1, 2, 10,
                                64, 0.f, nullptr) == GDN_ERR_ARG,
           "attn empty key set");
    EXPECT(gdn_attn_sink_window(P(A), P(A), nullptr, 10, nullptr, nullptr, 0, nullptr, nullptr, 0, P(A), 1, 2, 10,
                                64, 0.f, nullptr) == GDN_ERR_ARG,
           "attn sink values NULL");
    EXPECT(gdn_attn_sink_window(P(A), P(A), P(A), -1, nullptr, nullptr, 0, nullptr, nullptr, 0, P(A), 1, 2, 10, 64,
                                0.f, nullptr) == GDN_ERR_ARG,
           "attn negative length");
    EXPECT(gdn_attn_sink_window(P(A), P(A), P(A), 10, nullptr, nullptr, 0, nullptr, nullptr, 0, P(A), 1, 2, 0, 64,
                                0.f, nullptr) == GDN_OK,
           "attn Nq = 0 is a no-op");

    // ---- workspace queries over a grid of shapes, extremes included
    const int Bs[] = {0, 1, 2, 4, 65535, 65536, 0x7fffffff};
    const int Hs[] = {1, 16, 48, 4096};
    const int Ts[] = {0, 1, 63, 64, 65, 2640, 16384, 1 << 20, 0x7fffffff};
    const int Ds[] = {32, 64, 128, 48};
    const int Cs[] = {0, 16, 32, 64, 128};
    long checked = 0;
    for (int B : Bs)
        for (int H : Hs)
            for (int T : Ts)
                for (int dk : Ds)
                    for (int dv : Ds)
                        for (int C : Cs) {
                            const size_t w = gdn_workspace_bytes(B, H, T, dk, dv, C, nullptr);
                            const size_t b = gdn_bidir_workspace_bytes(B, H, T, dk, dv, C, nullptr);
                            EXPECT(w % 16 == 0 && b % 16 == 0, "alignment %d %d %d %d %d %d", B, H, T, dk, dv, C);
                            if (T == 0 || B == 0) EXPECT(w == 0 && b == 0, "empty shape needs nothing");
                            const size_t fw = gdn_framewise_workspace_bytes(B, H, T, 880, dk, dv, 0, nullptr);
                            EXPECT(fw % 16 == 0, "framewise alignment");
                            const size_t aw = gdn_attn_workspace_bytes(B, H, T, T, T, T, dk, nullptr);
                            EXPECT(aw % 16 == 0, "attn alignment");
                            ++checked;
                        }
    printf("%ld shapes queried, %d failures\n", checked, g_fail);
    return g_fail ? 1 : 0;
}
