// Drives the host-side call planning of the library (argument checks, frames per group,
// windows, workspace layout: linear_attention_video_gated_amd/csrc/gdn_plan.cpp) for a
// build with AddressSanitizer and UndefinedBehaviorSanitizer.  Checks the status codes and
// the workspace invariants the C ABI documents; exit status 0 when all hold.
#include <stdio.h>
#include <string.h>

#include "gdn_plan.hpp"

using namespace gdn;

static int fails = 0;
#define EXPECT(cond)                                                  \
    do {                                                              \
        if (!(cond)) {                                                \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #cond); \
            ++fails;                                                  \
        }                                                             \
    } while (0)

static gdn_dims_t dims(int B, int H, int F, int N, int d, int dtype = GDN_BF16, unsigned flags = GDN_F_NORMALIZE_K) {
    gdn_dims_t x;
    memset(&x, 0, sizeof x);
    x.B = B; x.H = H; x.n_frames = F; x.frame_len = N; x.d_k = d; x.d_v = d; x.dtype = dtype; x.flags = flags;
    return x;
}

int main() {
    Plan p;
    // status codes of bad dims
    EXPECT(check_dims(nullptr, GDN_ENTRY_FORWARD, &p, 256) == GDN_ERR_NULL);
    gdn_dims_t d = dims(1, 2, 3, 16, 32);
    d.dtype = 5;
    EXPECT(check_dims(&d, GDN_ENTRY_FORWARD, &p, 256) == GDN_ERR_DTYPE);
    d = dims(-1, 2, 3, 16, 32);
    EXPECT(check_dims(&d, GDN_ENTRY_FORWARD, &p, 256) == GDN_ERR_DIMS);
    d = dims(1, 2, 3, 0, 32);
    EXPECT(check_dims(&d, GDN_ENTRY_FORWARD, &p, 256) == GDN_ERR_DIMS);
    d = dims(1, 2, 3, 16, 48);
    EXPECT(check_dims(&d, GDN_ENTRY_FORWARD, &p, 256) == GDN_ERR_UNSUPPORTED);
    d = dims(1, 2, 3, 16, 32, GDN_BF16, GDN_F_RELU_QK);
    EXPECT(check_dims(&d, GDN_ENTRY_FORWARD, &p, 256) == GDN_ERR_UNSUPPORTED);
    d = dims(1, 2, 3, 16, 32, GDN_BF16, GDN_F_NORMALIZE_K);
    EXPECT(check_dims(&d, GDN_ENTRY_BLOCK_CAUSAL, &p, 256) == GDN_ERR_UNSUPPORTED);
    d = dims(1, 2, 3, 16, 32);
    d.window_units = -1;
    EXPECT(check_dims(&d, GDN_ENTRY_FORWARD, &p, 256) == GDN_ERR_DIMS);
    d = dims(70000, 1, 3, 16, 32);  // grid y extent
    EXPECT(check_dims(&d, GDN_ENTRY_FORWARD, &p, 256) == GDN_ERR_DIMS);
    d = dims(1, 1, 2000000000, 2000000000, 128);  // element count overflow
    EXPECT(check_dims(&d, GDN_ENTRY_FORWARD, &p, 256) == GDN_ERR_DIMS);

    // plans of many shapes: windows hold whole groups, the workspace does not grow with
    // the number of frames, every region lies inside the total
    const int ds[] = {16, 32, 64, 112, 128};
    const int Ns[] = {1, 16, 65, 390, 880, 4000};
    const int Fs[] = {1, 2, 7, 21, 240, 1000, 100000};
    const int BHs[][2] = {{1, 1}, {1, 20}, {16, 20}, {80, 20}};
    for (int entry = 0; entry < 4; ++entry)
        for (int dt = 0; dt < 2; ++dt)
            for (int di : ds)
                for (int N : Ns)
                    for (auto& bh : BHs) {
                        size_t first = 0;
                        for (int F : Fs) {
                            const unsigned fl = entry == GDN_ENTRY_BLOCK_CAUSAL ? GDN_F_RELU_QK : GDN_F_NORMALIZE_K;
                            d = dims(bh[0], bh[1], F, N, di, dt, fl);
                            Plan q;
                            const int rc = check_dims(&d, entry, &q, 256);
                            if (rc != GDN_OK) {  // only the overflow bound may refuse these
                                EXPECT(rc == GDN_ERR_DIMS);
                                continue;
                            }
                            EXPECT(q.nwin >= 1 && q.nfw >= 1 && q.G >= 1);
                            EXPECT((long long)q.nwin * q.nfw >= F);
                            EXPECT(entry == GDN_ENTRY_BLOCK_CAUSAL || q.nfw % q.G == 0 || q.nfw == F);
                            EXPECT(q.off_a <= q.off_b && q.off_b <= q.off_x && q.off_x <= q.off_ga &&
                                   q.off_ga <= q.off_gb && q.off_gb <= q.off_c && q.off_c <= q.off_carry &&
                                   q.off_carry <= q.total);
                            if (!first) first = q.total;
                            // bounded: one window holds at most max(8192, B H G) units
                            EXPECT(q.total <= first * (size_t)(8192 + 64 * bh[0] * bh[1]));
                        }
                    }
    // group choice: a single group for short calls, more groups than CUs never needed
    EXPECT(group_frames(20, 240, 880, 256) == 20);
    EXPECT(group_frames(320, 1, 880, 256) == 1);
    EXPECT(group_frames(1, 5, 100, 0) >= 1);
    // pointer helpers
    EXPECT(!misaligned(nullptr) && misaligned((void*)0x1008) && !misaligned((void*)0x1010));
    EXPECT(overlap((void*)0x1000, 16, (void*)0x100f, 1) && !overlap((void*)0x1000, 16, (void*)0x1010, 16));
    EXPECT(!overlap(nullptr, 16, (void*)0x1000, 16) && !overlap((void*)0x1000, 0, (void*)0x1000, 16));
    if (fails) fprintf(stderr, "%d check(s) failed\n", fails);
    else printf("plan sanitizer run: ok\n");
    return fails ? 1 : 0;
}
