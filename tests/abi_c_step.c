/* A training step driven from C through the C ABI, with device memory from
 * the HIP runtime (hipMalloc) and no Python or PyTorch in the process.  Run
 * by tests/test_gpu_c_client.py:
 *     c_client_step DIR BATCH LR d0 d1 ... dL
 * reads DIR/x.f32 [B*d0], DIR/labels.f32 [B*dL] and DIR/w<l>.f32 (raw
 * little-endian float32), runs mlp_grads and then mlp_train_step, writes
 * DIR/dw<l>.f32 and DIR/w<l>_out.f32, and prints the two losses. */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>

#include "mlp.h"

#define MAXL 16

static void die(const char* what, const char* msg) {
    fprintf(stderr, "%s: %s\n", what, msg);
    exit(1);
}

static float* read_f32(const char* dir, const char* name, size_t n) {
    char path[4096];
    FILE* f;
    float* h = (float*)malloc(n * sizeof(float));
    snprintf(path, sizeof path, "%s/%s", dir, name);
    f = fopen(path, "rb");
    if (!f || !h) die("open", path);
    if (fread(h, sizeof(float), n, f) != n) die("short read", path);
    fclose(f);
    return h;
}

static void write_f32(const char* dir, const char* name, const float* h, size_t n) {
    char path[4096];
    FILE* f;
    snprintf(path, sizeof path, "%s/%s", dir, name);
    f = fopen(path, "wb");
    if (!f || fwrite(h, sizeof(float), n, f) != n) die("write", path);
    fclose(f);
}

static void* to_device(const float* h, size_t n) {
    void* d = NULL;
    if (hipMalloc(&d, n * sizeof(float)) != hipSuccess) die("hipMalloc", "input");
    if (hipMemcpy(d, h, n * sizeof(float), hipMemcpyHostToDevice) != hipSuccess) die("hipMemcpy", "input");
    return d;
}

int main(int argc, char** argv) {
    int32_t dims[MAXL + 1];
    int L, B, l;
    float lr, loss_g = 0.f, loss_s = 0.f;
    const char* dir;
    mlp_config cfg;
    mlp_ctx* ctx = NULL;
    void* ws = NULL;
    size_t need;
    float *dx, *dt, *dw[MAXL], *dg[MAXL];
    float *hx, *ht;
    char name[64];

    if (argc < 6) die("usage", "c_client_step DIR BATCH LR d0 d1 ... dL");
    dir = argv[1];
    B = atoi(argv[2]);
    lr = (float)atof(argv[3]);
    L = argc - 5;
    if (L < 1 || L > MAXL) die("usage", "1..16 layers");
    for (l = 0; l <= L; ++l) dims[l] = atoi(argv[4 + l]);

    cfg.n_layers = L;
    cfg.dims = dims;
    cfg.batch = B;
    cfg.precision = MLP_F32;
    cfg.stream = NULL;
    need = mlp_workspace_bytes(&cfg);
    if (need == 0) die("mlp_workspace_bytes", mlp_last_error(NULL));
    if (hipMalloc(&ws, need) != hipSuccess) die("hipMalloc", "workspace");
    if (mlp_create(&cfg, ws, need, &ctx) != MLP_OK) die("mlp_create", mlp_last_error(NULL));

    hx = read_f32(dir, "x.f32", (size_t)B * dims[0]);
    ht = read_f32(dir, "labels.f32", (size_t)B * dims[L]);
    dx = (float*)to_device(hx, (size_t)B * dims[0]);
    dt = (float*)to_device(ht, (size_t)B * dims[L]);
    for (l = 0; l < L; ++l) {
        const size_t n = (size_t)dims[l] * dims[l + 1];
        float* h;
        snprintf(name, sizeof name, "w%d.f32", l);
        h = read_f32(dir, name, n);
        dw[l] = (float*)to_device(h, n);
        free(h);
        if (hipMalloc((void**)&dg[l], n * sizeof(float)) != hipSuccess) die("hipMalloc", "dW");
        if (mlp_set_params(ctx, l, dw[l]) != MLP_OK) die("mlp_set_params", mlp_last_error(ctx));
    }

    if (mlp_grads(ctx, dx, dt, dg, NULL, &loss_g) != MLP_OK) die("mlp_grads", mlp_last_error(ctx));
    if (mlp_train_step(ctx, dx, dt, lr, &loss_s) != MLP_OK) die("mlp_train_step", mlp_last_error(ctx));
    for (l = 0; l < L; ++l) {
        const size_t n = (size_t)dims[l] * dims[l + 1];
        float* h = (float*)malloc(n * sizeof(float));
        if (!h) die("malloc", "out");
        if (hipMemcpy(h, dg[l], n * sizeof(float), hipMemcpyDeviceToHost) != hipSuccess) die("hipMemcpy", "dW");
        snprintf(name, sizeof name, "dw%d.f32", l);
        write_f32(dir, name, h, n);
        if (mlp_read_params(ctx, l, dw[l]) != MLP_OK) die("mlp_read_params", mlp_last_error(ctx));
        if (hipDeviceSynchronize() != hipSuccess) die("hipDeviceSynchronize", "read");
        if (hipMemcpy(h, dw[l], n * sizeof(float), hipMemcpyDeviceToHost) != hipSuccess) die("hipMemcpy", "W");
        snprintf(name, sizeof name, "w%d_out.f32", l);
        write_f32(dir, name, h, n);
        free(h);
        hipFree(dg[l]);
        hipFree(dw[l]);
    }
    mlp_destroy(ctx);
    hipFree(dx);
    hipFree(dt);
    hipFree(ws);
    free(hx);
    free(ht);
    printf("loss_grads %.9g loss_step %.9g\n", loss_g, loss_s);
    return 0;
}
