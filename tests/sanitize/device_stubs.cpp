// Stand-ins for the library's device-side functions (defined in the .hip
// sources, which this host-only sanitizer build does not compile).  The
// driver only makes calls that the C ABI rejects before reaching them, so
// each one aborts if it is ever reached.
#include <cstdio>
#include <cstdlib>

#include "ocq_internal.h"

namespace ocq {

[[noreturn]] static void unreachable(const char* what) {
  std::fprintf(stderr, "device entry %s reached in a host-only build\n", what);
  std::abort();
}

int launch_forward(const Plan&, const FwdArgs&) { unreachable("launch_forward"); }
void set_fused_requant(int) {}
int diag_stream_read(const void*, size_t, void*, int, void*) { unreachable("diag_stream_read"); }
int diag_window_read(const void*, size_t, int, void*, int, void*) { unreachable("diag_window_read"); }
size_t diag_mfma_rate_flops(int, int) { unreachable("diag_mfma_rate_flops"); }
int diag_mfma_rate(int, float*, int, void*) { unreachable("diag_mfma_rate"); }
int diag_empty(void*) { unreachable("diag_empty"); }
int diag_mfma_dot(int, const uint8_t*, const uint8_t*, int, int, int, float*, void*) { unreachable("diag_mfma_dot"); }
// as in a library built without phase stamps
int lg_phase_copy(void*, size_t) { return -1; }
int pc_phase_copy(void*, size_t) { return -1; }
int q_phase_copy(void*, size_t) { return -1; }

}  // namespace ocq
