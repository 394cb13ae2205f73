// Error reporting and the fixed-stride expert blob format.
//
// One expert = one contiguous record so that fetching it is one copy: the
// pages repack routed experts into fixed-stride blobs so one read is one
// fetch ([xix] how-it-works paragraph; [digest] "Core Mechanics").  The
// order and alignment of the sections inside a blob are this library's own
// choice: the three packed-word sections first, then the three (scale, bias)
// sections, each 256-byte aligned, the record padded to 4096 bytes.
#include <cstring>
#include <string>

#include "common.h"

namespace moe {

static thread_local std::string g_last_error;

int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error.clear(); }

static int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

bool blob_layout(const moe_qshape& s, moe_blob_layout* out) {
  if (s.group != 64) return fail(MOE_E_INVAL, "group must be 64 (got %d)", s.group), false;
  if (s.bits != 4 && s.bits != 8) return fail(MOE_E_INVAL, "bits must be 4 or 8 (got %d)", s.bits), false;
  if (s.hidden <= 0 || s.inter <= 0 || s.hidden % 64 || s.inter % 64)
    return fail(MOE_E_INVAL, "hidden (%d) and inter (%d) must be positive multiples of 64",
                s.hidden, s.inter), false;
  const int64_t H = s.hidden, I = s.inter;
  // rows x packed bytes per row, for gate [I,H], up [I,H], down [H,I]
  const int64_t rows[3] = {I, I, H};
  const int64_t cols[3] = {H, H, I};
  int64_t off = 0;
  for (int m = 0; m < 3; ++m) {
    out->q_off[m] = off;
    out->q_bytes[m] = rows[m] * cols[m] * s.bits / 8;
    off = round_up(off + out->q_bytes[m], 256);
  }
  for (int m = 0; m < 3; ++m) {
    out->sb_off[m] = off;
    out->sb_bytes[m] = rows[m] * (cols[m] / s.group) * 4;
    off = round_up(off + out->sb_bytes[m], 256);
  }
  out->bytes = off;
  out->stride = round_up(off, 4096);
  return true;
}

}  // namespace moe

extern "C" {

const char* moe_last_error(void) { return moe::g_last_error.c_str(); }

int32_t moe_blob_layout_get(const moe_qshape* shape, moe_blob_layout* out) {
  MOE_REQUIRE(shape && out, "null argument");
  moe::clear_error();
  return moe::blob_layout(*shape, out) ? MOE_OK : MOE_E_INVAL;
}

int32_t moe_blob_pack(const moe_qshape* shape, const moe_qmatrix_host* gate,
                      const moe_qmatrix_host* up, const moe_qmatrix_host* down,
                      void* blob_host) {
  MOE_REQUIRE(shape && gate && up && down && blob_host, "null argument");
  moe_blob_layout lay;
  if (!moe::blob_layout(*shape, &lay)) return MOE_E_INVAL;
  const moe_qmatrix_host* mats[3] = {gate, up, down};
  uint8_t* dst = static_cast<uint8_t*>(blob_host);
  std::memset(dst, 0, static_cast<size_t>(lay.stride));
  const int64_t rows[3] = {shape->inter, shape->inter, shape->hidden};
  const int64_t cols[3] = {shape->hidden, shape->hidden, shape->inter};
  for (int m = 0; m < 3; ++m) {
    MOE_REQUIRE(mats[m]->q && mats[m]->s && mats[m]->b, "null matrix part %d", m);
    std::memcpy(dst + lay.q_off[m], mats[m]->q, static_cast<size_t>(lay.q_bytes[m]));
    uint32_t* sb = reinterpret_cast<uint32_t*>(dst + lay.sb_off[m]);
    const int64_t n = rows[m] * (cols[m] / shape->group);
    for (int64_t i = 0; i < n; ++i)
      sb[i] = uint32_t(mats[m]->s[i]) | (uint32_t(mats[m]->b[i]) << 16);
  }
  return MOE_OK;
}

}  // extern "C"
