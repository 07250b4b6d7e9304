// host_stubs.cpp -- stand-ins for the library's device-side entry points,
// linked with the host-only units (C ABI checks and planning) into a
// sanitizer build that runs on the CPU: every launch reports failure, and
// the planner's row counts are those of the real kernels.  Test
// infrastructure only; never part of the product library.
#include <cstdint>

#include "attn_launch.h"
#include "gdn_launch.h"
#include "proj_launch.h"

namespace attn {
int launch_bf16(const LaunchArgs &, int, void *) { return 1; }
int launch_f32(const LaunchArgs &, int, void *) { return 1; }
int launch_decode_bf16(const DecodeArgs &, int, void *) { return 1; }
int rows_per_workgroup_bf16(int) { return 128; }
int rows_per_workgroup_bf16_halves(int) { return 64; }
int rows_per_workgroup_f32(int) { return 128; }
int decode_scratch(void *, void **ptr) {
  *ptr = nullptr;
  return 1;
}
int work_tickets(LaunchArgs &a, void *) {
  a.tickets = nullptr;
  a.ticket_from = a.total_items;
  return 0;
}
}  // namespace attn

namespace gdn {
int launch_gdn(const GdnArgs &, void *) { return 1; }
}  // namespace gdn

namespace proj {
int launch_dequantize_int8(const int8_t *, const float *, void *, int64_t, int64_t, void *) {
  return 1;
}
}  // namespace proj
