// Kernel-launch entry points for the host-only sanitizer build of the contract
// and planner: the driver never gets past the host checks, so reaching any of
// these is itself a failure.
#include <cstdio>
#include <cstdlib>

#include "../../varlen_flash_attention_fa_amd/csrc/fa_internal.h"

namespace fa {

int launch_fwd(const Plan&, const FwdParams&, void*, void*, void*) {
    std::fprintf(stderr, "launch_fwd reached in the host-only build\n");
    std::abort();
}
const char* last_hip_error() { return "host-only build"; }
int launch_kv_append(const AppendParams&, void*, void*, void*) {
    std::fprintf(stderr, "launch_kv_append reached in the host-only build\n");
    std::abort();
}
const char* last_append_error() { return "host-only build"; }
int static_scratch(void*, void**, size_t*) {
    std::fprintf(stderr, "static_scratch reached in the host-only build\n");
    std::abort();
}

}  // namespace fa
