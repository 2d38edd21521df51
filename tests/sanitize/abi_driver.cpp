// abi_driver.cpp -- calls every entry point of include/kda.h with fake,
// far-apart device addresses and valid or invalid arguments, on a host with
// or without a GPU, under AddressSanitizer and UndefinedBehaviorSanitizer.
// Every call stops at a host-side check or at the device check (no GPU: the
// launch functions are stubs that abort if reached).  Test infrastructure only.
#include <stdint.h>
#include <stdio.h>

#include "kda.h"

namespace {

int failures = 0;

void expect(int got, int want, int want2, const char *what) {
    if (got != want && got != want2) {
        fprintf(stderr, "%s: got %d, want %d or %d\n", what, got, want, want2);
        ++failures;
    }
}

uintptr_t next_addr = uintptr_t(1) << 40;
void *fake() {  // 16-byte aligned, 64 GiB apart
    void *p = reinterpret_cast<void *>(next_addr);
    next_addr += uintptr_t(64) << 30;
    return p;
}

}  // namespace

int main() {
    const int D = KDA_ERR_DEVICE;
    void *q = fake(), *k = fake(), *v = fake(), *out = fake();
    float *g = static_cast<float *>(fake()), *b = static_cast<float *>(fake());
    float *s0 = static_cast<float *>(fake()), *s1 = static_cast<float *>(fake());
    float *snap = static_cast<float *>(fake());
    const int32_t *cu = static_cast<const int32_t *>(fake());
    void *ws = fake();
    // kda_chunk_fwd
    expect(kda_chunk_fwd(q, k, v, g, b, s0, nullptr, out, s1, 2, 100, 3, 128, 128, 0, 1, nullptr),
           D, KDA_OK, "chunk valid");
    expect(kda_chunk_fwd(nullptr, k, v, g, b, s0, nullptr, out, s1, 2, 100, 3, 128, 128, 0, 1,
                         nullptr), KDA_ERR_NULL, KDA_ERR_NULL, "chunk null q");
    expect(kda_chunk_fwd(q, k, v, g, b, s0, nullptr, out, s1, -1, 100, 3, 128, 128, 0, 1, nullptr),
           KDA_ERR_SHAPE, KDA_ERR_SHAPE, "chunk batch<0");
    expect(kda_chunk_fwd(q, k, v, g, b, s0, nullptr, out, s1, 2, 100, 3, 96, 96, 0, 1, nullptr),
           KDA_ERR_UNSUPPORTED, KDA_ERR_UNSUPPORTED, "chunk d=96");
    expect(kda_chunk_fwd(static_cast<char *>(q) + 8, k, v, g, b, s0, nullptr, out, s1, 2, 100, 3,
                         128, 128, 0, 1, nullptr), KDA_ERR_ALIGN, KDA_ERR_ALIGN, "chunk align");
    expect(kda_chunk_fwd(q, k, v, g, b, s0, nullptr, q, s1, 2, 100, 3, 128, 128, 0, 1, nullptr),
           KDA_ERR_ALIAS, KDA_ERR_ALIAS, "chunk alias");
    expect(kda_chunk_fwd(q, k, v, g, b, s0, cu, out, s1, 1, 100, 3, 128, 128, 4, 1, nullptr), D,
           KDA_OK, "chunk packed");
    expect(kda_chunk_fwd(q, k, v, g, b, s0, nullptr, out, s0, 2, 100, 3, 64, 64, 0, 0, nullptr), D,
           KDA_OK, "chunk in place fp32");
    // snapshots and scalar gate
    expect(kda_chunk_fwd_snapshots(q, k, v, g, b, s0, nullptr, out, s1, snap, 64, 2, 1, 128, 3,
                                   128, 128, 0, 1, nullptr), D, KDA_OK, "snapshots valid");
    expect(kda_chunk_fwd_snapshots(q, k, v, g, b, s0, nullptr, out, s1, snap, 48, 2, 1, 128, 3,
                                   128, 128, 0, 1, nullptr), KDA_ERR_UNSUPPORTED,
           KDA_ERR_UNSUPPORTED, "snapshots interval");
    expect(kda_chunk_fwd_scalar_gate(q, k, v, g, b, s0, nullptr, out, s1, 2, 100, 3, 128, 128, 0,
                                     1, nullptr), D, KDA_OK, "scalar gate valid");
    // segmented, with a workspace and with the fixed scratch
    const int64_t need = kda_chunk_fwd_segmented_workspace_size(4096, 3, 128, 4);
    expect(need > 0, 1, 1, "segmented size");
    expect(kda_chunk_fwd_segmented(q, k, v, g, b, s0, out, s1, 4096, 3, 128, 128, 4, 1, ws, need,
                                   nullptr), D, KDA_OK, "segmented valid");
    expect(kda_chunk_fwd_segmented(q, k, v, g, b, s0, out, s1, 4096, 3, 128, 128, 4, 1, ws,
                                   need - 1, nullptr), KDA_ERR_SHAPE, KDA_ERR_SHAPE,
           "segmented small workspace");
    expect(kda_chunk_fwd_segmented_noalloc(q, k, v, g, b, s0, out, s1, 4096, 3, 128, 128, 4, 1,
                                           nullptr), D, KDA_OK, "noalloc valid");
    expect(kda_chunk_fwd_segmented_noalloc(q, k, v, g, b, s0, out, s1, 1 << 20, 32, 128, 128, 16,
                                           1, nullptr), KDA_ERR_SCRATCH, KDA_ERR_SCRATCH,
           "noalloc beyond the scratch");
    // backward
    void *dq = fake(), *dk = fake(), *dv = fake(), *dout = fake();
    float *dg = static_cast<float *>(fake()), *db = static_cast<float *>(fake());
    float *ds0 = static_cast<float *>(fake()), *dsT = static_cast<float *>(fake());
    const int64_t bneed = kda_chunk_bwd_workspace_size(200, 2, 3, 128);
    expect(kda_chunk_bwd(q, k, v, g, b, s0, nullptr, dout, dsT, dq, dk, dv, dg, db, ds0, 2, 100,
                         3, 128, 128, 0, 1, ws, bneed, nullptr), D, KDA_OK, "bwd valid");
    expect(kda_chunk_bwd(q, k, v, g, b, s0, nullptr, dout, dsT, dq, dk, dv, dg, db, ds0, 2, 100,
                         3, 128, 128, 0, 1, ws, bneed - 1, nullptr), KDA_ERR_SHAPE,
           KDA_ERR_SHAPE, "bwd small workspace");
    expect(kda_chunk_bwd(q, k, v, g, b, s0, nullptr, dout, dsT, q, dk, dv, dg, db, ds0, 2, 100,
                         3, 128, 128, 0, 1, ws, bneed, nullptr), KDA_ERR_ALIAS, KDA_ERR_ALIAS,
           "bwd alias");
    // decode
    expect(kda_decode_step(q, k, v, g, b, s0, out, 256, 96, 128, 128, 1, nullptr), D, KDA_OK,
           "decode valid");
    expect(kda_decode_step(q, k, v, g, b, s0, s0, 256, 96, 128, 128, 1, nullptr), KDA_ERR_ALIAS,
           KDA_ERR_ALIAS, "decode alias");
    expect(kda_decode_step_scalar_gate(q, k, v, g, b, s0, out, 0, 96, 128, 128, 1, nullptr),
           KDA_OK, KDA_OK, "decode empty");
    // status strings and version
    for (int s = -9; s <= 1; ++s)
        if (!kda_status_string(s)[0]) ++failures;
    expect(kda_abi_version(), KDA_ABI_VERSION, KDA_ABI_VERSION, "version");
    printf("abi driver: %d failures\n", failures);
    return failures ? 1 : 0;
}
