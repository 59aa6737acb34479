// bc_clock.hpp -- per-phase clocks of the GEMV and attention kernels.
//
// Only a build with -DBC_PHASE_CLOCKS (libbc_clk.so) records them; in the
// library itself every stamp compiles to nothing and no launch gets a clock
// buffer.  A work-group's thread 0 keeps its stamps in scalar registers and
// stores them at its end into kClockSlots 64-bit entries of the launch's
// slice of a buffer the caller registered (bc_phase_clocks_begin):
//   [0] real-time counter (100 MHz) at the start, [1] at the end,
//   [2] shader clock at the start, [3..12] shader clock at phase ends (which
//   phases depends on the kernel; 0 where a phase did not run), [13] shader
//   clock at the end, [14] XCC id, [15] hardware id (CU, SIMD, wave).
// Stamps are taken by the first wave only: they show when that wave reached
// each point, and a barrier right before a stamp makes it the work-group's.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bc {

#ifdef BC_PHASE_CLOCKS
constexpr bool kPhaseClocks = true;
#else
constexpr bool kPhaseClocks = false;
#endif
constexpr int kClockSlots = 16;

struct PhaseClock {
  unsigned long long t[kPhaseClocks ? kClockSlots : 1];

  __device__ __forceinline__ void begin() {
    if constexpr (kPhaseClocks) {
#pragma unroll
      for (int i = 0; i < kClockSlots; ++i) t[i] = 0;
      t[0] = __builtin_amdgcn_s_memrealtime();
      t[2] = __builtin_amdgcn_s_memtime();
    }
  }
  __device__ __forceinline__ void stamp(int i) {
    if constexpr (kPhaseClocks) t[i] = __builtin_amdgcn_s_memtime();
  }
  // a stamp that waits for `v` (a loaded value) first: the time it arrived
  __device__ __forceinline__ void stamp_after(int i, float v) {
    if constexpr (kPhaseClocks) {
      unsigned long long c;
      asm volatile("s_memtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(c) : "v"(v));
      t[i] = c;
    }
  }
  // stores the stamps of work-group `group` (thread 0) when dst is set
  __device__ __forceinline__ void end(unsigned long long* dst, size_t group) {
    if constexpr (kPhaseClocks) {
      t[13] = __builtin_amdgcn_s_memtime();
      t[1] = __builtin_amdgcn_s_memrealtime();
      t[14] = unsigned(__builtin_amdgcn_s_getreg((3 << 11) | 20));    // XCC_ID, 4 bits
      t[15] = unsigned(__builtin_amdgcn_s_getreg((31 << 11) | 4));    // HW_ID
      if (dst != nullptr && threadIdx.x == 0) {
#pragma unroll
        for (int i = 0; i < kClockSlots; ++i) dst[group * kClockSlots + i] = t[i];
      }
    }
  }
};

// Host: the clock slice for a launch of `groups` work-groups, or NULL (the
// library itself, or no buffer registered, or the buffer full).  kind and
// a..d describe the launch for bc_phase_clocks_info.
unsigned long long* clock_take(size_t groups, int kind, int a, int b, int c, int d);
enum ClockKind : int { CLOCK_GEMV = 1, CLOCK_ATTN = 2 };

}  // namespace bc
