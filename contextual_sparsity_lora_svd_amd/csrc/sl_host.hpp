// Host-side helpers of the C ABI: error state, validation, layout tables and
// workspace planning.  No device memory is ever allocated here.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "sl_common.hpp"

namespace sl {

void set_error(const char* fmt, ...);
const char* last_error();

#define SL_FAIL(code, ...)            \
  do {                                \
    ::sl::set_error(__VA_ARGS__);     \
    return code;                      \
  } while (0)

#define SL_HIP(call)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess)                                                              \
      SL_FAIL(SL_ERR_HIP, "%s failed: %s (%s:%d)", #call, hipGetErrorString(e_),       \
              __FILE__, __LINE__);                                                     \
  } while (0)

sl_status check_arch();
int device_cus();   // compute units of the current device (0 when none)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The gather-GEMM addresses its operands with 32-bit element offsets, and its
// LDS-DMA loads with 32-bit byte offsets of 2-byte elements: every matrix it
// reads or writes (token-major activations, weights, compact buffers) must
// hold fewer than 2^31 elements.  Checked on the host before any launch.
constexpr long long kMaxOperandElems = (1LL << 31) - 1;
inline sl_status check_extent(const char* what, long long rows, long long cols) {
  if (rows > 0 && cols > 0 && rows > kMaxOperandElems / cols)
    SL_FAIL(SL_ERR_RANGE, "%s holds %lld x %lld elements; at most 2^31 - 1 are supported", what, rows, cols);
  return SL_OK;
}

// Validate and tabulate a sequence layout.
sl_status build_seqtab(const sl_layout* lay, SeqTab& st);

// Bump allocator for offsets inside a caller buffer (256-byte aligned regions).
struct Bump {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = (off + bytes + 255) & ~size_t(255);
    return o;
  }
};

// Fork and join with a side stream, for work of a call that does not depend on
// the launches it may overlap.  Each caller stream of each device gets a side
// stream of its own (default priority, non-blocking), created at its first
// fork, so calls on independent streams never wait for each other; the pair
// keeps one fork and one join event, re-recorded by every fork and join
// (device-scope release, no timing).  begin(): the side stream waits for everything
// enqueued on `main` so far.  end(): `main` waits for everything enqueued on
// the side stream so far, so the call's work is again ordered on `main`.
// refork(): the side stream waits again for everything enqueued on `main` so
// far.  Each fork or join point leaves `main` idle about 5 us on MI355X (an
// event record or wait between two kernels), so calls use few of them.
// While `main` is being captured into a graph, begin() makes `side` = `main`
// and all of these are no-ops: the captured work stays on one stream.
struct SideFork {
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  sl_status begin(hipStream_t main);
  sl_status end(hipStream_t main);
  sl_status refork(hipStream_t main);
};

// Optional per-launch timing: when enabled (sl_timer_enable), selected launches
// are bracketed by HIP events on their stream and attributed to a slot.
enum TimerSlot {
  TS_ESTIMATE = 0, TS_SELECT, TS_GU_FWD, TS_DOWN_FWD, TS_DH_BWD, TS_DX_BWD, TS_QKV_FWD, TS_O_FWD,
  TS_DA_BWD, TS_DXQKV_BWD, TS_LORA, TS_NSLOTS
};
bool timer_on();
void timer_begin(int slot, hipStream_t s);
void timer_end(int slot, hipStream_t s);

inline int pow2_rm(int R) { return R <= 8 ? 8 : R <= 16 ? 16 : R <= 32 ? 32 : 64; }
inline int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

inline dim3 grid1d(long long n, int threads = 256) { return dim3((unsigned)((n + threads - 1) / threads)); }

}  // namespace sl
