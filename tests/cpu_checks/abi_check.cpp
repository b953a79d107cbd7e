// Host-side checks of libdrr's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_cpu_checks.py): every
// entry point is called with invalid arguments (and empty sizes) that its
// host validation must reject -- or accept as a no-op -- before any HIP call.
// Host arrays are heap allocations of exactly the documented length, so a
// read past spacing[3], K[9], ras2ijk[16] or the transfer knots is reported.
// Device pointers are dummies that no path here dereferences.
// Exit status 0 when every status matches; failures are printed.
#include <stdio.h>
#include <string.h>

#include <vector>

#include "../../include/drr.h"

static int g_fail = 0;

static void expect(int got, int want, const char* what)
{
    const char* err = drr_last_error();
    if (got != want) {
        ++g_fail;
        fprintf(stderr, "FAIL %s: status %d, expected %d (%s)\n", what, got, want, err);
        return;
    }
    if (want != DRR_OK && (err == nullptr || err[0] == '\0')) {
        ++g_fail;
        fprintf(stderr, "FAIL %s: status %d with no error message\n", what, got);
    }
}

template <int N>
struct HostArr {
    std::vector<float> v;
    HostArr(std::initializer_list<float> x) : v(x) { v.resize(N); }
    float* p() { return v.data(); }
};

int main()
{
    void* D = reinterpret_cast<void*>(0x1000);        // never dereferenced
    float* Df = static_cast<float*>(D);
    std::vector<float> sp{1.0f, 1.0f, 1.0f}, sp_bad{1.0f, 0.0f, 1.0f};
    std::vector<float> K{500, 0, 32, 0, 500, 32, 0, 0, 1}, K_sing{1, 2, 3, 2, 4, 6, 0, 0, 1};
    std::vector<float> ras{1, 0, 0, 31.5f, 0, 1, 0, 31.5f, 0, 0, 1, 31.5f, 0, 0, 0, 1};
    std::vector<float> ras_bad{1, 0, 0, 0, 1, 0, 0, 0, 0, 0, 1, 0, 0, 0, 0, 1};   // rows 0, 1 parallel
    std::vector<float> xp{-1000, 0, 1500}, yp{0, 0.02f, 0.05f}, xp_bad{0, 0, 1};

    if (drr_abi_version() != DRR_ABI_VERSION) {
        fprintf(stderr, "FAIL abi version\n");
        ++g_fail;
    }
    for (int s = -1; s <= 5; ++s)
        if (drr_status_string(s) == nullptr || strlen(drr_status_string(s)) == 0) ++g_fail;

    // workspace queries: invalid sizes give 0, valid ones are 256-byte multiples
    const int qs[][9] = {{64, 64, 64, 0, 1, 64, 64, 128, 0},   {256, 256, 256, 1, 16, 200, 200, 256, 0},
                         {128, 128, 128, 0, 360, 256, 384, 256, 1}, {8, 8, 8, 0, 64, 16, 16, 8, 2},
                         {0, 8, 8, 0, 1, 4, 4, 8, 0},          {8, 8, 8, 7, 1, 4, 4, 8, 0},
                         {8, 8, 8, 0, -1, 4, 4, 8, 1},         {8, 8, 8, 0, 1, 4, 4, 0, 2}};
    for (const auto& q : qs) {
        const size_t n = drr_workspace_bytes(q[0], q[1], q[2], q[3], q[4], q[5], q[6], q[7], q[8]);
        if (n % 256 != 0) {
            ++g_fail;
            fprintf(stderr, "FAIL workspace %zu not a 256-byte multiple\n", n);
        }
    }
    for (int fb = 0; fb < 3; ++fb)
        for (int mode = 0; mode < 3; ++mode)
            for (int clip = 0; clip < 2; ++clip)
                if (drr_render_workspace_bytes(2, 3, 20, 21, 22, 1, 4, 30, 31, 40, mode, clip, 3, fb) %
                        256 != 0)
                    ++g_fail;
    if (drr_render_workspace_bytes(2, 3, 20, 21, 22, 1, 5, 30, 31, 40, 0, 0, 0, 0) != 0) ++g_fail;

    // forward (and the no-allocation forward)
    expect(drr_forward(D, 0, 0, 8, 8, sp.data(), K.data(), Df, 1, 4, 4, 8, 0, Df, nullptr, nullptr, 0, nullptr),
           DRR_ERR_INVALID_ARGUMENT, "forward nz = 0");
    expect(drr_forward(D, 0, 8, 8, 20000, sp.data(), K.data(), Df, 1, 4, 4, 8, 0, Df, nullptr, nullptr, 0, nullptr),
           DRR_ERR_UNSUPPORTED, "forward nx too large");
    expect(drr_forward(D, 3, 8, 8, 8, sp.data(), K.data(), Df, 1, 4, 4, 8, 0, Df, nullptr, nullptr, 0, nullptr),
           DRR_ERR_INVALID_ARGUMENT, "forward dtype");
    expect(drr_forward(D, 0, 8, 8, 8, sp_bad.data(), K.data(), Df, 1, 4, 4, 8, 0, Df, nullptr, nullptr, 0, nullptr),
           DRR_ERR_INVALID_ARGUMENT, "forward spacing 0");
    expect(drr_forward(D, 0, 8, 8, 8, sp.data(), K_sing.data(), Df, 1, 4, 4, 8, 0, Df, nullptr, nullptr, 0, nullptr),
           DRR_ERR_INVALID_ARGUMENT, "forward singular K");
    expect(drr_forward(D, 0, 8, 8, 8, sp.data(), K.data(), Df, 1, 4, 4, 8, 2, Df, nullptr, nullptr, 0, nullptr),
           DRR_ERR_INVALID_ARGUMENT, "forward mode 2");
    expect(drr_forward(D, 0, 8, 8, 8, sp.data(), K.data(), Df, 65536, 256, 256, 8, 0, Df, nullptr, nullptr, 0, nullptr),
           DRR_ERR_UNSUPPORTED, "forward > 2^31 rays");
    expect(drr_forward(D, 0, 8, 8, 8, sp.data(), K.data(), Df, 64, 16, 16, 8, 0, Df, nullptr, nullptr, 0, nullptr),
           DRR_ERR_WORKSPACE_TOO_SMALL, "forward workspace");
    expect(drr_forward(D, 0, 8, 8, 8, sp.data(), K.data(), nullptr, 0, 4, 4, 8, 0, nullptr, nullptr, nullptr, 0, nullptr),
           DRR_OK, "forward empty");
    expect(drr_forward_reuse(D, 0, 8, 8, 8, sp_bad.data(), K.data(), Df, 1, 4, 4, 8, 0, Df, nullptr, nullptr, 0, nullptr),
           DRR_ERR_INVALID_ARGUMENT, "reuse forward spacing 0");
    expect(drr_forward_reuse(D, 0, 8, 8, 8, sp.data(), K.data(), Df, 64, 16, 16, 8, 0, Df, nullptr, nullptr, 0, nullptr),
           DRR_ERR_WORKSPACE_TOO_SMALL, "reuse forward workspace");
    expect(drr_forward_reuse(D, 0, 8, 8, 8, sp.data(), K.data(), nullptr, 0, 4, 4, 8, 0, nullptr, nullptr, nullptr, 0, nullptr),
           DRR_OK, "reuse forward empty");
    expect(drr_forward_no_alloc(D, 0, 512, 512, 512, sp.data(), K.data(), Df, 64, 256, 256, 256, 0, Df, nullptr, nullptr),
           DRR_ERR_UNSUPPORTED, "no-alloc forward beyond the scratch");
    expect(drr_forward_no_alloc(nullptr, 0, 8, 8, 8, sp.data(), K.data(), Df, 1, 4, 4, 8, 0, Df, nullptr, nullptr),
           DRR_ERR_INVALID_ARGUMENT, "no-alloc forward volume NULL");
    expect(drr_forward_no_alloc(D, 0, 8, 8, 8, sp.data(), K.data(), nullptr, 0, 4, 4, 8, 0, nullptr, nullptr, nullptr),
           DRR_OK, "no-alloc forward empty");

    // volume backward
    expect(drr_backward_volume(8, 8, 8, sp.data(), K.data(), Df, 1, 4, 4, 8, 0, Df, nullptr, Df, nullptr, 0, nullptr),
           DRR_ERR_INVALID_ARGUMENT, "backward BL without line integral");
    expect(drr_backward_volume(8, 8, 8, sp.data(), K.data(), Df, 1, 4, 4, 8, 1, Df, nullptr, nullptr, nullptr, 0, nullptr),
           DRR_ERR_INVALID_ARGUMENT, "backward grad NULL");
    expect(drr_backward_volume(8, 8, 8, sp.data(), K.data(), Df, 1, 4, 4, 8, 1, Df, nullptr, Df, nullptr, 0, nullptr),
           DRR_ERR_WORKSPACE_TOO_SMALL, "backward records workspace");
    expect(drr_backward_volume(8, 8, 8, sp.data(), K.data(), Df, 1, 4, 4, 8, 1, Df, nullptr, Df,
                               reinterpret_cast<void*>(0x1004), 4096, nullptr),
           DRR_ERR_INVALID_ARGUMENT, "backward misaligned workspace");
    expect(drr_backward_volume(8, 8, 8, sp.data(), K.data(), Df, 1, 4, 4, -3, 1, Df, nullptr, Df, nullptr, 0, nullptr),
           DRR_ERR_INVALID_ARGUMENT, "backward n_samples");

    // pose backward, Siddon pair
    expect(drr_backward_pose(D, 0, 8, 8, 8, sp.data(), K.data(), Df, 1, 4, 4, 8, 0, Df, Df, nullptr, 0, nullptr),
           DRR_ERR_WORKSPACE_TOO_SMALL, "pose backward workspace");
    expect(drr_backward_pose(D, 0, 8, 8, 8, sp.data(), K.data(), Df, 1, 4, 4, 8, 0, nullptr, Df, D, 4096, nullptr),
           DRR_ERR_INVALID_ARGUMENT, "pose backward grad_out NULL");
    expect(drr_backward_pose_reuse(D, 0, 8, 8, 8, sp.data(), K.data(), Df, 1, 4, 4, 8, 0, Df, Df, nullptr, 0, nullptr),
           DRR_ERR_WORKSPACE_TOO_SMALL, "reuse pose backward workspace");
    expect(drr_backward_pose_reuse(D, 0, 8, 8, 8, sp.data(), K.data(), Df, 1, 4, 4, 8, 0, nullptr, Df, D, 4096, nullptr),
           DRR_ERR_INVALID_ARGUMENT, "reuse pose backward grad_out NULL");
    expect(drr_forward_siddon(D, 0, 8, 8, 8, sp_bad.data(), K.data(), Df, 1, 4, 4, 0, Df, nullptr, nullptr),
           DRR_ERR_INVALID_ARGUMENT, "siddon forward spacing");
    expect(drr_backward_volume_siddon(8, 8, 8, sp.data(), K.data(), Df, 1, 4, 4, 0, Df, nullptr, Df, nullptr),
           DRR_ERR_INVALID_ARGUMENT, "siddon backward BL without line integral");

    // render: views not a multiple of volumes, transfer knots not increasing,
    // half-given transfer function, bad clip
    expect(drr_render(D, 0, 2, 1, 8, 8, 8, sp.data(), K.data(), Df, 3, 4, 4, 8, 0, 1.0f, 0, 30.0f,
                      nullptr, nullptr, 0, Df, nullptr, nullptr, 0, nullptr),
           DRR_ERR_INVALID_ARGUMENT, "render views per volume");
    expect(drr_render(D, 0, 1, 1, 8, 8, 8, sp.data(), K.data(), Df, 1, 4, 4, 8, 0, 1.0f, 0, 30.0f,
                      xp_bad.data(), yp.data(), 3, Df, nullptr, nullptr, 0, nullptr),
           DRR_ERR_INVALID_ARGUMENT, "render transfer knots");
    expect(drr_render(D, 0, 1, 1, 8, 8, 8, sp.data(), K.data(), Df, 1, 4, 4, 8, 0, 1.0f, 0, 30.0f,
                      xp.data(), nullptr, 3, Df, nullptr, nullptr, 0, nullptr),
           DRR_ERR_INVALID_ARGUMENT, "render half transfer");
    expect(drr_render(D, 0, 1, 1, 8, 8, 8, sp.data(), K.data(), Df, 1, 4, 4, 8, 0, 1.0f, 5, 30.0f,
                      nullptr, nullptr, 0, Df, nullptr, nullptr, 0, nullptr),
           DRR_ERR_INVALID_ARGUMENT, "render clip");
    expect(drr_render_reuse(D, 0, 2, 1, 8, 8, 8, sp.data(), K.data(), Df, 3, 4, 4, 8, 0, 1.0f, 0,
                            30.0f, nullptr, nullptr, 0, Df, nullptr, nullptr, 0, nullptr),
           DRR_ERR_INVALID_ARGUMENT, "reuse render views per volume");
    expect(drr_render_reuse(D, 0, 1, 1, 8, 8, 8, sp.data(), K.data(), Df, 1, 4, 4, 8, 0, 1.0f, 5,
                            30.0f, nullptr, nullptr, 0, Df, nullptr, nullptr, 0, nullptr),
           DRR_ERR_INVALID_ARGUMENT, "reuse render clip");
    expect(drr_render_backward_pose_reuse(D, 0, 1, 1, 8, 8, 8, sp.data(), K.data(), Df, 1, 4, 4,
                                          8, 0, 1.0f, 0, 30.0f, nullptr, nullptr, 0, Df, Df,
                                          nullptr, 0, nullptr),
           DRR_ERR_WORKSPACE_TOO_SMALL, "reuse render pose workspace");
    expect(drr_render_backward_volume(D, 0, 1, 1, 8, 8, 8, sp.data(), K.data(), Df, 1, 4, 4, 8, 2,
                                      1.0f, 0, 30.0f, nullptr, nullptr, 0, Df, nullptr, Df, Df,
                                      nullptr, 0, nullptr),
           DRR_ERR_INVALID_ARGUMENT, "render backward compositing without image");
    // the near/far pose backward reads a zero-padded copy: a workspace of the
    // view sums alone is too small
    expect(drr_render_backward_pose(D, 0, 1, 1, 8, 8, 8, sp.data(), K.data(), Df, 1, 4, 4, 8, 2,
                                    1.0f, 1, 30.0f, nullptr, nullptr, 0, Df, Df, D, 256, nullptr),
           DRR_ERR_WORKSPACE_TOO_SMALL, "render pose backward near/far workspace");

    // cameras
    std::vector<float> Kout(9);
    expect(drr_intrinsics_from_fov(20.0f, 1024, 1024, Kout.data()), DRR_OK, "fov");
    if (!(Kout[0] > 2903.0f && Kout[0] < 2904.5f)) {
        ++g_fail;
        fprintf(stderr, "FAIL fov focal %g\n", Kout[0]);
    }
    expect(drr_intrinsics_from_fov(190.0f, 1024, 1024, Kout.data()), DRR_ERR_INVALID_ARGUMENT, "fov range");
    expect(drr_poses_from_view_matrices(Df, 1, ras_bad.data(), 64, 64, 64, Df, nullptr, nullptr),
           DRR_ERR_INVALID_ARGUMENT, "view matrices non-orthogonal ras2ijk");
    expect(drr_view_matrices_backward(Df, 1, nullptr, 64, 64, 64, Df, Df, nullptr),
           DRR_ERR_INVALID_ARGUMENT, "view matrix backward ras2ijk NULL");
    (void)ras;

    // noise surrogate
    expect(drr_poisson_surrogate(Df, Df, -1, 1e4f, Df, nullptr), DRR_ERR_INVALID_ARGUMENT, "noise n");
    expect(drr_poisson_surrogate(Df, Df, 10, 0.0f, Df, nullptr), DRR_ERR_INVALID_ARGUMENT, "noise i0");
    expect(drr_poisson_surrogate(nullptr, nullptr, 0, 1e4f, nullptr, nullptr), DRR_OK, "noise empty");

    if (g_fail) {
        fprintf(stderr, "%d ABI check(s) failed\n", g_fail);
        return 1;
    }
    printf("all ABI host checks passed\n");
    return 0;
}
