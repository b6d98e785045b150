/* A C99 caller of the public C ABI (include/mhc.h): compiled and run by
 * tests/test_c_abi.py on the host.  Only calls that return before touching a
 * device are made -- version, strings, defaults, empty batches and argument
 * errors -- so no GPU is needed.  Prints one line per failed check and exits
 * with the number of failures. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mhc.h"

static int failures = 0;

#define CHECK(cond)                                             \
    do {                                                        \
        if (!(cond)) {                                          \
            printf("FAILED line %d: %s\n", __LINE__, #cond);    \
            ++failures;                                         \
        }                                                       \
    } while (0)

/* aligned addresses that are never dereferenced: every call that gets them
 * fails validation first */
#define FAKE(off) ((float*)(uintptr_t)(0x10000u + (off)))

int main(void)
{
    mhc_proj_opts o;
    mhc_layer_args la;

    CHECK(mhc_abi_version() == 4);
    CHECK(strcmp(mhc_status_string(MHC_OK), "ok") == 0);
    CHECK(strcmp(mhc_status_string(MHC_ERR_INVALID_ARGUMENT), "invalid argument") == 0);
    CHECK(mhc_last_error() != NULL);

    CHECK(mhc_proj_opts_default(&o) == MHC_OK);
    CHECK(o.solver == MHC_SOLVER_NEWTON && o.max_iters == -1 && o.warm_sweeps == -1);
    CHECK(o.tol > 0.9e-6f && o.tol < 1.1e-6f);
    CHECK(mhc_proj_opts_default(NULL) == MHC_ERR_INVALID_ARGUMENT);

    /* empty batches are no-ops */
    CHECK(mhc_birkhoff_fwd(NULL, NULL, 0, NULL, NULL, NULL) == MHC_OK);
    CHECK(mhc_birkhoff_bwd(NULL, NULL, NULL, 0, NULL) == MHC_OK);
    CHECK(mhc_birkhoff_fwd_n(NULL, NULL, 0, 3, NULL, NULL, NULL) == MHC_OK);
    CHECK(mhc_birkhoff_bwd_recompute(NULL, NULL, NULL, 0, NULL, NULL) == MHC_OK);
    CHECK(mhc_birkhoff_fwd_bwd(NULL, NULL, NULL, NULL, 0, NULL, NULL, NULL) == MHC_OK);

    /* argument errors */
    CHECK(mhc_birkhoff_fwd(FAKE(0), FAKE(0), -1, NULL, NULL, NULL) == MHC_ERR_INVALID_ARGUMENT);
    CHECK(mhc_birkhoff_fwd(NULL, FAKE(0), 5, NULL, NULL, NULL) == MHC_ERR_INVALID_ARGUMENT);
    CHECK(mhc_birkhoff_fwd(FAKE(4), FAKE(4096), 5, NULL, NULL, NULL) == MHC_ERR_INVALID_ARGUMENT);
    CHECK(mhc_birkhoff_fwd(FAKE(0), FAKE(64), 5, NULL, NULL, NULL) == MHC_ERR_INVALID_ARGUMENT);
    o.max_iters = -2;
    CHECK(mhc_birkhoff_fwd(FAKE(0), FAKE(0), 5, &o, NULL, NULL) == MHC_ERR_INVALID_ARGUMENT);
    o.max_iters = -1;
    /* size limits */
    CHECK(mhc_birkhoff_bwd(FAKE(0), FAKE(8192), FAKE(16384), MHC_MAX_BATCH + 1, NULL) ==
          MHC_ERR_INVALID_ARGUMENT);
    CHECK(strstr(mhc_last_error(), "out of range") != NULL);
    CHECK(mhc_stream_mix(FAKE(0), FAKE(8192), NULL, FAKE(16384), MHC_MAX_TOKENS + 1, 4, 64, NULL,
                         NULL) == MHC_ERR_INVALID_ARGUMENT);
    CHECK(strstr(mhc_last_error(), "out of range") != NULL);
    CHECK(mhc_birkhoff_bwd(FAKE(0), NULL, FAKE(0), 3, NULL) == MHC_ERR_INVALID_ARGUMENT);
    CHECK(mhc_birkhoff_bwd_recompute(FAKE(0), FAKE(8192), FAKE(64), 3, NULL, NULL) ==
          MHC_ERR_INVALID_ARGUMENT);
    /* fused: P may alias logits, but not grad_P */
    CHECK(mhc_birkhoff_fwd_bwd(FAKE(0), FAKE(8192), FAKE(8192), FAKE(16384), 3, NULL, NULL,
                               NULL) == MHC_ERR_INVALID_ARGUMENT);
    CHECK(mhc_birkhoff_fwd_bwd(FAKE(0), FAKE(8192), FAKE(16384), FAKE(64), 3, NULL, NULL,
                               NULL) == MHC_ERR_INVALID_ARGUMENT);
    CHECK(mhc_birkhoff_fwd_n(FAKE(0), FAKE(0), 5, 9, NULL, NULL, NULL) == MHC_ERR_UNSUPPORTED);
    CHECK(mhc_birkhoff_bwd_n(FAKE(0), FAKE(0), FAKE(0), 5, 0, NULL) == MHC_ERR_UNSUPPORTED);
    CHECK(mhc_stream_mix(FAKE(0), FAKE(8192), NULL, FAKE(16384), 4, 5, 64, NULL, NULL) ==
          MHC_ERR_UNSUPPORTED);
    CHECK(mhc_stream_mix(FAKE(0), FAKE(8192), NULL, FAKE(16384), 4, 4, 60, NULL, NULL) ==
          MHC_ERR_INVALID_ARGUMENT);

    /* layer: workspace size and argument errors */
    CHECK(mhc_layer_workspace_bytes(65536, 4, 7168) > 0);
    CHECK(mhc_layer_workspace_bytes(16, 3, 64) == -1);
    memset(&la, 0, sizeof la);
    CHECK(mhc_layer_fwd(NULL, NULL) == MHC_ERR_INVALID_ARGUMENT);
    la.T = 16;
    la.n = 4;
    la.C = 100; /* not a multiple of 64 */
    la.eps = 1e-6f;
    CHECK(mhc_layer_fwd(&la, NULL) != MHC_OK);
    CHECK(mhc_layer_bwd(&la, NULL) != MHC_OK);

    if (failures == 0) printf("c abi ok\n");
    return failures;
}
