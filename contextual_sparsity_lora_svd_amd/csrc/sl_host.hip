// Error state, device checks and layout tables of the C ABI.
#include "sl_host.hpp"

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

sl_status check_arch() {
  int dev = 0;
  SL_HIP(hipGetDevice(&dev));
  static int checked[64] = {0};   // 0 unknown, 1 ok, 2 wrong arch (benign race: same answer)
  if (dev >= 0 && dev < 64 && checked[dev] == 1) return SL_OK;
  hipDeviceProp_t prop;
  SL_HIP(hipGetDeviceProperties(&prop, dev));
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < 64) checked[dev] = ok ? 1 : 2;
  if (!ok)
    SL_FAIL(SL_ERR_UNSUPPORTED_ARCH, "device %d is %s; this library is built for gfx950", dev,
            prop.gcnArchName);
  return SL_OK;
}

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

}  // namespace sl

extern "C" {

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
