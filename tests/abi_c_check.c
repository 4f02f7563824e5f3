/* Compiled as C99 by tests/test_c_header_cpu.py: include/mlp.h must be a
 * plain C header, and the host-only entry points must link and answer
 * without a GPU (argument checks, workspace sizes, status names). */
#include <stdio.h>
#include <string.h>

#include "mlp.h"

static int fails = 0;
#define CHECK(c)                                              \
    do {                                                      \
        if (!(c)) {                                           \
            fprintf(stderr, "check failed: %s\n", #c);        \
            ++fails;                                          \
        }                                                     \
    } while (0)

int main(void) {
    const int32_t dims[4] = {1024, 4096, 4096, 1000};
    mlp_config cfg;
    mlp_ctx* ctx = NULL;
    size_t need;
    unsigned char buf[64];
    int32_t n_layers = 0;

    memset(&cfg, 0, sizeof cfg);
    cfg.n_layers = 3;
    cfg.dims = dims;
    cfg.batch = 4096;
    cfg.precision = MLP_F32;
    cfg.stream = NULL;

    CHECK(mlp_abi_version() == MLP_ABI_VERSION);
    need = mlp_workspace_bytes(&cfg);
    CHECK(need > 0 && need % 256 == 0);
    CHECK(mlp_workspace_bytes(NULL) == 0);
    CHECK(strcmp(mlp_status_string(MLP_ERR_GUARD), "MLP_ERR_GUARD") == 0);
    CHECK(strcmp(mlp_status_string((mlp_status)99), "MLP_ERR_UNKNOWN") == 0);
    /* no workspace: refused before any device work */
    CHECK(mlp_create(&cfg, NULL, need, &ctx) == MLP_ERR_WORKSPACE && ctx == NULL);
    CHECK(strlen(mlp_last_error(NULL)) > 0);
    CHECK(mlp_set_debug(NULL, MLP_DEBUG_SYNC | MLP_DEBUG_GUARDS) == MLP_ERR_ARG);
    CHECK(mlp_optimizer_bytes(&cfg, MLP_OPT_ADAM) > 0);
    CHECK(mlp_optimizer_bytes(&cfg, MLP_OPT_SGD) == 0);
    memset(buf, 0, sizeof buf);
    CHECK(mlp_checkpoint_info(buf, sizeof buf, &n_layers, NULL, NULL, NULL) == MLP_ERR_ARG);
    printf("ok: abi %d, workspace %zu bytes\n", (int)mlp_abi_version(), need);
    return fails != 0;
}
