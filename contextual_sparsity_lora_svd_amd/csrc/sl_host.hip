// Error state, device checks and layout tables of the C ABI.
#include "sl_host.hpp"
#include "sl_gemm.hpp"

#include <atomic>
#include <mutex>
#include <vector>

namespace sl {

static thread_local std::string g_err;

void set_error(const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
}

const char* last_error() { return g_err.c_str(); }

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  static std::atomic<int> cus[64];   // per device, filled on first use (zero-initialised)
  if (dev >= 0 && dev < 64) {
    const int c = cus[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
  return prop.multiProcessorCount;
}

sl_status check_arch() {
  int dev = 0;
  SL_HIP(hipGetDevice(&dev));
  static std::atomic<int> checked[64];   // 0 unknown, 1 ok, 2 wrong arch
  if (dev >= 0 && dev < 64 && checked[dev].load(std::memory_order_relaxed) == 1) return SL_OK;
  hipDeviceProp_t prop;
  SL_HIP(hipGetDeviceProperties(&prop, dev));
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < 64) checked[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  if (!ok)
    SL_FAIL(SL_ERR_UNSUPPORTED_ARCH, "device %d is %s; this library is built for gfx950", dev,
            prop.gcnArchName);
  return SL_OK;
}

namespace {
// Side streams, one per (device, caller stream), created on first use and
// kept until the process ends.  Past kMaxSide caller streams per process a
// call keeps all of its work on the caller's stream.
constexpr int kMaxSide = 256;
// ev[0] links the caller's stream to the side stream (fork), ev[1] the side
// stream back (join).  A wait takes the event's latest record at the time of
// the wait, so each event is simply re-recorded by the next fork or join.
// The events carry no timing and release to device scope only: both streams
// run on one device, and the host never inspects them.
struct SideEntry { int dev; hipStream_t main; hipStream_t side; hipEvent_t ev[2]; };
std::mutex g_side_mu;
SideEntry g_side[kMaxSide];
int g_nside = 0;

sl_status link_streams(hipStream_t from, hipStream_t to, hipEvent_t ev) {
  SL_HIP(hipEventRecord(ev, from));
  SL_HIP(hipStreamWaitEvent(to, ev, 0));
  return SL_OK;
}
}  // namespace

sl_status SideFork::begin(hipStream_t main) {
  // a stream being captured into a graph keeps all of the call's work: the
  // graph then needs no cross-stream events
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  SL_HIP(hipStreamIsCapturing(main, &cs));
  if (cs != hipStreamCaptureStatusNone) {
    side = main;
    return SL_OK;
  }
  int dev = 0;
  SL_HIP(hipGetDevice(&dev));
  {
    std::lock_guard<std::mutex> lk(g_side_mu);
    side = main;
    for (int i = 0; i < g_nside; ++i)
      if (g_side[i].dev == dev && g_side[i].main == main) {
        side = g_side[i].side;
        ev_fork = g_side[i].ev[0];
        ev_join = g_side[i].ev[1];
        if (link_streams(main, side, ev_fork) != SL_OK) return SL_ERR_HIP;
        return SL_OK;
      }
    if (g_nside < kMaxSide) {
      SideEntry e{dev, main, nullptr, {nullptr, nullptr}};
      const unsigned fl = hipEventDisableTiming | hipEventReleaseToDevice;
      SL_HIP(hipStreamCreateWithFlags(&e.side, hipStreamNonBlocking));
      SL_HIP(hipEventCreateWithFlags(&e.ev[0], fl));
      SL_HIP(hipEventCreateWithFlags(&e.ev[1], fl));
      g_side[g_nside++] = e;
      side = e.side;
      ev_fork = e.ev[0];
      ev_join = e.ev[1];
      return link_streams(main, side, ev_fork);
    }
  }
  return SL_OK;   // no side stream left: the call keeps its work on `main`
}

sl_status SideFork::end(hipStream_t main) { return side == main ? SL_OK : link_streams(side, main, ev_join); }

sl_status SideFork::refork(hipStream_t main) { return side == main ? SL_OK : link_streams(main, side, ev_fork); }


sl_status build_seqtab(const sl_layout* lay, SeqTab& st) {
  if (!lay) SL_FAIL(SL_ERR_NULL, "layout is NULL");
  if (!lay->ctx_len) SL_FAIL(SL_ERR_NULL, "layout.ctx_len is NULL");
  if (lay->batch < 1 || lay->batch > SL_MAX_SEQS)
    SL_FAIL(SL_ERR_RANGE, "batch %d outside [1, %d]", lay->batch, SL_MAX_SEQS);
  if (lay->seq_len < 1) SL_FAIL(SL_ERR_RANGE, "seq_len %d < 1", lay->seq_len);
  if ((long long)lay->batch * lay->seq_len > (1LL << 30))
    SL_FAIL(SL_ERR_RANGE, "too many tokens");
  std::memset(&st, 0, sizeof(st));
  st.nseq = lay->batch;
  st.L = lay->seq_len;
  int cp = 0, op = 0;
  for (int b = 0; b < lay->batch; ++b) {
    const int c = lay->ctx_len[b];
    if (c < 0 || c > lay->seq_len)
      SL_FAIL(SL_ERR_RANGE, "ctx_len[%d] = %d outside [0, %d]", b, c, lay->seq_len);
    st.ctx[b] = c;
    st.ctx_pre[b] = cp;
    st.out_pre[b] = op;
    cp += c;
    op += lay->seq_len - c;
  }
  st.ctx_pre[lay->batch] = cp;
  st.out_pre[lay->batch] = op;
  st.T_ctx = cp;
  st.T_out = op;
  return SL_OK;
}

// ---- launch timing ---------------------------------------------------------
struct TimerState {
  bool on = false;
  std::vector<hipEvent_t> ev;      // pairs (start, stop)
  std::vector<int> slot;
  size_t used = 0;
  uint32_t mask = ~0u;             // slots recorded
};
static thread_local TimerState g_timer;   // per calling thread
static thread_local int g_pending_slot = -1;

bool timer_on() { return g_timer.on; }

void timer_begin(int slot, hipStream_t s) {
  if (slot < 0) return;   // untimed launch: leaves a pending measurement alone
  if (!g_timer.on || !((g_timer.mask >> slot) & 1u) || 2 * (g_timer.used + 1) > g_timer.ev.size()) {
    g_pending_slot = -1;
    return;
  }
  g_pending_slot = slot;
  hipEventRecord(g_timer.ev[2 * g_timer.used], s);
}

void timer_end(int slot, hipStream_t s) {
  if (slot < 0 || !g_timer.on || g_pending_slot != slot) return;
  hipEventRecord(g_timer.ev[2 * g_timer.used + 1], s);
  g_timer.slot[g_timer.used] = slot;
  ++g_timer.used;
  g_pending_slot = -1;
}

}  // namespace sl

extern "C" {

/* Diagnostics (not part of the computation): bracket the library's main
 * launches with HIP events.  Enable with room for max_launches launches; read
 * per-slot totals after synchronising; disable frees the events. */
int sl_timer_enable(int max_launches) {
  using namespace sl;
  for (hipEvent_t e : g_timer.ev) hipEventDestroy(e);
  g_timer.ev.clear();
  g_timer.slot.clear();
  g_timer.used = 0;
  g_timer.on = false;
  g_timer.mask = ~0u;
  if (max_launches <= 0) return 0;
  g_timer.ev.resize(2 * (size_t)max_launches);
  g_timer.slot.resize(max_launches);
  for (auto& e : g_timer.ev)
    // timing only: no system-scope fence at the record (the host reads the
    // events after synchronizing the stream)
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return (int)SL_ERR_HIP;
  g_timer.on = true;
  return 0;
}

void sl_timer_select(uint32_t slot_mask) { sl::g_timer.mask = slot_mask; }

int sl_gemm_config(int variants) {
  const int prev = sl::g_gemm_variants;
  if (variants >= 0) sl::g_gemm_variants = variants & (sl::GV_WIDE | sl::GV_TALL | sl::GV_TALL_ALWAYS);
  return prev;
}

void sl_timer_reset(void) { sl::g_timer.used = 0; }

/* Total milliseconds and launch count recorded for a slot since the last reset. */
int sl_timer_read(int slot, double* total_ms, int* count) {
  using namespace sl;
  double t = 0;
  int n = 0;
  for (size_t i = 0; i < g_timer.used; ++i) {
    if (g_timer.slot[i] != slot) continue;
    float ms = 0;
    if (hipEventSynchronize(g_timer.ev[2 * i + 1]) != hipSuccess) return (int)SL_ERR_HIP;
    if (hipEventElapsedTime(&ms, g_timer.ev[2 * i], g_timer.ev[2 * i + 1]) != hipSuccess)
      return (int)SL_ERR_HIP;
    t += ms;
    ++n;
  }
  if (total_ms) *total_ms = t;
  if (count) *count = n;
  return 0;
}

int sl_abi_version(void) { return SL_ABI_VERSION; }

const char* sl_status_string(sl_status s) {
  switch (s) {
    case SL_OK: return "ok";
    case SL_ERR_NULL: return "null pointer";
    case SL_ERR_ALIGN: return "misaligned pointer";
    case SL_ERR_SHAPE: return "bad shape";
    case SL_ERR_DTYPE: return "bad dtype or criterion";
    case SL_ERR_RANGE: return "argument out of range";
    case SL_ERR_WORKSPACE: return "buffer too small";
    case SL_ERR_UNSUPPORTED_ARCH: return "unsupported device";
    case SL_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* sl_last_error(void) { return sl::last_error(); }

}  // extern "C"
