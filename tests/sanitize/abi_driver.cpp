// Calls every entry point of libkda's C ABI (include/kda.h) with arguments the
// host validation must reject, and the size queries, in a build whose host
// code has AddressSanitizer and UndefinedBehaviorSanitizer: every call below
// returns before any HIP call, so no GPU is needed.  Exit code 0 means every
// call gave the expected status and the sanitizers saw nothing.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "kda.h"

static int fails = 0;
static void expect(int got, int want, const char *what) {
    if (got != want) {
        std::fprintf(stderr, "FAILED %s: status %d, expected %d (%s)\n", what, got, want, kda_last_error());
        ++fails;
    } else if (want != KDA_OK && std::strlen(kda_last_error()) == 0) {
        std::fprintf(stderr, "FAILED %s: no message\n", what);
        ++fails;
    }
}

int main() {
    // fake, never dereferenced device pointers: validation fails before any use
    auto P = [](uintptr_t i) { return reinterpret_cast<void *>(i * 0x100000); };
    auto F = [&](uintptr_t i) { return static_cast<float *>(P(i)); };
    const float inf = INFINITY;

    if (kda_abi_version() != KDA_ABI_VERSION) {
        std::fprintf(stderr, "FAILED abi version %d\n", kda_abi_version());
        ++fails;
    }
    // kda_chunk_fwd
    expect(kda_chunk_fwd(P(1), P(2), P(3), F(4), F(5), nullptr, P(6), nullptr, 1, 8, 2, 3, 32, 32, 0.f, 0, 1,
                         nullptr, 0, nullptr), KDA_EINVAL, "chunk HV % H");
    expect(kda_chunk_fwd(P(1), P(2), P(3), F(4), F(5), nullptr, P(6), nullptr, 1, 8, 2, 2, 48, 32, 0.f, 0, 1,
                         nullptr, 0, nullptr), KDA_EUNSUPPORTED, "chunk K");
    expect(kda_chunk_fwd(P(1), P(2), P(3), F(4), F(5), nullptr, P(6), nullptr, 1, 8, 2, 2, 32, 32, inf, 0, 1,
                         nullptr, 0, nullptr), KDA_EINVAL, "chunk scale");
    expect(kda_chunk_fwd(P(1), P(2), P(3), F(4), F(5), nullptr, P(6), nullptr, 1, 8, 2, 2, 32, 32, 0.f, 0, 1,
                         nullptr, -5, nullptr), KDA_EINVAL, "chunk workspace bytes");
    expect(kda_chunk_fwd(P(1), P(2), P(3), F(4), F(5), nullptr, P(3), nullptr, 1, 8, 2, 2, 32, 32, 0.f, 0, 1,
                         nullptr, 0, nullptr), KDA_EINVAL, "chunk out overlaps v");
    expect(kda_chunk_fwd(P(1), P(2), P(3), F(4), F(5), nullptr, P(6), nullptr, 1 << 20, 1 << 20, 128, 128, 128,
                         128, 0.f, 0, 1, nullptr, 0, nullptr), KDA_EINVAL, "chunk overflow");
    expect(static_cast<int>(kda_chunk_fwd_workspace_size(1, 8192, 96, 96, 128, 128, 0, 1)), KDA_OK, "workspace size");
    expect(static_cast<int>(kda_chunk_fwd_workspace_size(1, 8, 2, 2, 32, 32, 64, 1)), -1, "workspace size chunk");
    // kda_chunk_fwd_gated
    expect(kda_chunk_fwd_gated(P(1), P(2), P(3), F(4), F(5), F(6), F(7), -6.f, nullptr, nullptr, 0.f, P(9),
                               nullptr, 1, 8, 2, 2, 32, 32, 0.f, 0, 1, nullptr, 0, nullptr),
           KDA_EINVAL, "gated lower bound");
    expect(kda_chunk_fwd_gated(P(1), P(2), P(3), F(4), F(5), F(6), F(7), -5.f, nullptr, nullptr, 0.f, P(9),
                               nullptr, 1, 8, 2, 2, 32, 32, 0.f, 0, 0, nullptr, 0, nullptr),
           KDA_EUNSUPPORTED, "gated fp32");
    // kda_chunk_fwd_snapshots
    expect(kda_chunk_fwd_snapshots(P(1), P(2), P(3), F(4), F(5), nullptr, P(6), nullptr, F(7), 48, 1, 64, 2, 2, 32,
                                   32, 0.f, 0, 1, nullptr, 0, nullptr), KDA_EINVAL, "snapshots every");
    // kda_recurrent_fwd
    expect(kda_recurrent_fwd(nullptr, P(2), P(3), F(4), F(5), nullptr, P(6), nullptr, 1, 8, 2, 2, 32, 32, 0.f, 1,
                             nullptr), KDA_EINVAL, "recurrent null q");
    // kda_recurrent_bwd and its no-alloc variant
    expect(static_cast<int>(kda_recurrent_bwd_workspace_size(1, 8, 2, 3, 32, 32)), -1, "bwd workspace size");
    expect(kda_recurrent_bwd(P(1), P(2), P(3), F(4), F(5), nullptr, P(6), nullptr, P(7), P(8), P(9), F(10), F(11),
                             nullptr, 1, 8, 2, 2, 32, 32, 0.f, 1, P(12), 16, nullptr), KDA_EINVAL, "bwd small workspace");
    expect(kda_recurrent_bwd_noalloc(P(1), P(2), P(3), F(4), F(5), nullptr, P(6), nullptr, P(7), P(8), P(9), F(10),
                                     F(11), nullptr, 1, 8192, 96, 96, 128, 128, 0.f, 1, nullptr),
           KDA_EUNSUPPORTED, "noalloc past the scratch");
    // kda_prefill_prologue
    kda_decode_prologue pro{};
    pro.conv_weight = F(20);
    pro.conv_kernel = 9;
    expect(kda_prefill_prologue(P(1), F(2), F(3), &pro, P(4), P(5), P(6), F(7), F(8), 1, 8, 2, 2, 32, 32, 1, nullptr),
           KDA_EUNSUPPORTED, "prologue conv width");
    expect(kda_prefill_prologue(P(1), F(2), F(3), nullptr, P(4), P(5), P(6), nullptr, F(8), 1, 8, 2, 2, 32, 32, 1,
                                nullptr), KDA_EINVAL, "prologue half gate stage");
    // kda_output_gate
    expect(kda_output_gate(P(1), P(2), P(2), 8, 32, 1e-6f, 1, nullptr), KDA_EINVAL, "output gate y overlaps gate");
    expect(kda_output_gate(P(1), P(2), P(3), 8, 32, -1.f, 1, nullptr), KDA_EINVAL, "output gate eps");
    // kda_decode_step
    kda_decode_prologue dp{};
    dp.gate_mode = KDA_GATE_BOUNDED;
    expect(kda_decode_step(P(1), F(2), F(3), F(4), P(5), &dp, 2, 2, 2, 32, 32, 0.f, 1, nullptr), KDA_EINVAL,
           "decode gate without A_log");
    expect(kda_decode_step(P(1), F(2), F(3), F(4), P(5), nullptr, 2, 2, 2, 32, 32, 0.f, 7, nullptr),
           KDA_EUNSUPPORTED, "decode dtype");
    std::printf("abi driver: %d failure(s)\n", fails);
    return fails ? 1 : 0;
}
