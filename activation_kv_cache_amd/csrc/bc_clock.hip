// bc_clock.hip -- host side of the per-phase clocks (bc_clock.hpp): the
// registered buffer, the launches that took a slice of it, and the C entry
// points.  In the library itself the entry points report BC_ERR_UNSUPPORTED
// and no launch takes a slice.
#include <mutex>

#include "bc_clock.hpp"
#include "bc_internal.hpp"

namespace bc {

namespace {

constexpr int kClockMaxLaunches = 16384;

struct ClockLaunch {
  int kind, a, b, c, d;
  size_t groups, offset;   // in work-groups and in 64-bit entries
};

std::mutex g_clock_mu;
unsigned long long* g_clock_buf = nullptr;
size_t g_clock_cap = 0, g_clock_used = 0;
int g_clock_n = 0;
ClockLaunch g_clock_launch[kClockMaxLaunches];

}  // namespace

unsigned long long* clock_take(size_t groups, int kind, int a, int b, int c, int d) {
  if constexpr (!kPhaseClocks) {
    return nullptr;
  } else {
    std::lock_guard<std::mutex> lk(g_clock_mu);
    const size_t need = groups * kClockSlots;
    if (!g_clock_buf || g_clock_n >= kClockMaxLaunches || g_clock_used + need > g_clock_cap) return nullptr;
    g_clock_launch[g_clock_n++] = ClockLaunch{kind, a, b, c, d, groups, g_clock_used};
    unsigned long long* p = g_clock_buf + g_clock_used;
    g_clock_used += need;
    return p;
  }
}

}  // namespace bc

using namespace bc;

extern "C" int bc_phase_clocks_begin(void* buf, size_t bytes) {
  if (!kPhaseClocks) return set_error(BC_ERR_UNSUPPORTED, "bc_phase_clocks_begin: a build without phase clocks");
  if (buf != nullptr && (reinterpret_cast<uintptr_t>(buf) & 7))
    return set_error(BC_ERR_INVALID, "bc_phase_clocks_begin: buffer not 8-byte aligned");
  std::lock_guard<std::mutex> lk(g_clock_mu);
  g_clock_buf = static_cast<unsigned long long*>(buf);
  g_clock_cap = buf ? bytes / sizeof(unsigned long long) : 0;
  g_clock_used = 0;
  g_clock_n = 0;
  return BC_OK;
}

extern "C" int bc_phase_clocks_count(void) {
  if (!kPhaseClocks) return set_error(BC_ERR_UNSUPPORTED, "bc_phase_clocks_count: a build without phase clocks");
  std::lock_guard<std::mutex> lk(g_clock_mu);
  return g_clock_n;
}

extern "C" int bc_phase_clocks_info(int i, long long* out7) {
  if (!kPhaseClocks) return set_error(BC_ERR_UNSUPPORTED, "bc_phase_clocks_info: a build without phase clocks");
  if (out7 == nullptr) return set_error(BC_ERR_INVALID, "bc_phase_clocks_info: NULL output");
  std::lock_guard<std::mutex> lk(g_clock_mu);
  if (i < 0 || i >= g_clock_n) return set_error(BC_ERR_INVALID, "bc_phase_clocks_info: launch %d of %d", i, g_clock_n);
  const ClockLaunch& l = g_clock_launch[i];
  out7[0] = l.kind;
  out7[1] = l.a;
  out7[2] = l.b;
  out7[3] = l.c;
  out7[4] = l.d;
  out7[5] = static_cast<long long>(l.groups);
  out7[6] = static_cast<long long>(l.offset);
  return BC_OK;
}
