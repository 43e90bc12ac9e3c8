// C-ABI entry points of libattn.so (declared in include/attn.h).
//
// Host side only: argument validation (no HIP call is made before every
// check has passed), choice of the kernel instance and the launch on the
// caller's stream.  The operation itself is documented in attn.h.

#include <cmath>
#include <cstdint>

#include "attn.h"
#include "attn_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

// byte ranges [a, a + na) and [b, b + nb); sizes in 128-bit so no product can wrap
bool overlaps(const void* a, unsigned __int128 na, const void* b, unsigned __int128 nb) {
  if (na == 0 || nb == 0) return false;
  const unsigned __int128 a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

int fwd(attn::DType dt, const void* q, const void* k, const void* v, void* out, int B, int h, int Tq,
        int Tk, int d_k, int d_v, float scale, int mask_kind, const int32_t* key_lens,
        hipStream_t stream) {
  if (B < 0 || h < 0 || Tq < 0 || Tk < 0 || d_k < 0 || d_v < 0) return ATTN_ERR_SHAPE;
  if (d_k != d_v) return ATTN_ERR_SHAPE;
  if (d_k != 64 && d_k != 128) return ATTN_ERR_HEADDIM;
  if (mask_kind & ~(ATTN_MASK_CAUSAL | ATTN_MASK_KEYPAD)) return ATTN_ERR_MASK;
  const bool causal = (mask_kind & ATTN_MASK_CAUSAL) != 0;
  const bool keypad = (mask_kind & ATTN_MASK_KEYPAD) != 0;
  if (keypad && key_lens == nullptr) return ATTN_ERR_MASK;
  if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
  if (B == 0 || h == 0 || Tq == 0) return ATTN_OK;  // nothing to compute
  if (q == nullptr || out == nullptr) return ATTN_ERR_NULL;
  if (Tk > 0 && (k == nullptr || v == nullptr)) return ATTN_ERR_NULL;
  if (misaligned(q, 16) || misaligned(out, 16) || (Tk > 0 && (misaligned(k, 16) || misaligned(v, 16))))
    return ATTN_ERR_ALIGN;
  if (keypad && misaligned(key_lens, 4)) return ATTN_ERR_ALIGN;

  const int64_t bm = attn::rows_per_block(dt, d_k);
  const int64_t bh = static_cast<int64_t>(B) * h;
  const int64_t n_qtiles = (Tq + bm - 1) / bm;
  const int64_t n_wg = bh * n_qtiles;  // B, h < 2^31 and n_qtiles < 2^25: no overflow
  if (n_wg > 0x7fffffffLL) return ATTN_ERR_TOO_LARGE;

  typedef unsigned __int128 u128;
  const u128 es = dt == attn::DType::F32 ? 4 : 2;
  const u128 nq = (u128)bh * Tq * d_k * es, nkv = (u128)bh * Tk * d_k * es, no = (u128)bh * Tq * d_v * es;
  if (overlaps(out, no, q, nq) || overlaps(out, no, k, nkv) || overlaps(out, no, v, nkv))
    return ATTN_ERR_ALIAS;

  attn::Params p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = out;
  p.key_lens = keypad ? key_lens : nullptr;
  p.B = B;
  p.H = h;
  p.Tq = Tq;
  p.Tk = Tk;
  // |scale| * log2(e), kept >= 1e-30 so that masked (-inf) scores always map to
  // exp2(-inf) = 0; for scale = 0 every exp2 argument then rounds to 0 and the
  // weights are exactly uniform, as for a true zero.
  p.scale_log2 = static_cast<float>(std::fmax(std::fabs(static_cast<double>(scale)) * 1.4426950408889634, 1e-30));
  p.neg = scale < 0.f ? 1 : 0;
  p.n_qtiles = static_cast<int>(n_qtiles);
  p.n_wg = static_cast<int>(n_wg);
  const hipError_t e = attn::launch_fwd(p, dt, d_k, causal, keypad, stream);
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int h, int Tq, int Tk,
             int d_k, int d_v, float scale, int mask_kind, const int32_t* key_lens, hipStream_t stream) {
  return fwd(attn::DType::BF16, q, k, v, out, B, h, Tq, Tk, d_k, d_v, scale, mask_kind, key_lens, stream);
}

int attn_fwd_f32(const void* q, const void* k, const void* v, void* out, int B, int h, int Tq, int Tk,
                 int d_k, int d_v, float scale, int mask_kind, const int32_t* key_lens,
                 hipStream_t stream) {
  return fwd(attn::DType::F32, q, k, v, out, B, h, Tq, Tk, d_k, d_v, scale, mask_kind, key_lens, stream);
}

const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer argument";
    case ATTN_ERR_SHAPE: return "bad shape (negative dimension or d_k != d_v)";
    case ATTN_ERR_HEADDIM: return "unsupported head size (supported: 64, 128)";
    case ATTN_ERR_MASK: return "bad mask_kind bits, or key padding without key_lens";
    case ATTN_ERR_ALIAS: return "out overlaps q, k or v";
    case ATTN_ERR_ALIGN: return "misaligned pointer (tensors need 16 bytes, key_lens 4)";
    case ATTN_ERR_SCALE: return "scale is not finite";
    case ATTN_ERR_TOO_LARGE: return "too many work-groups for one launch";
    case ATTN_ERR_HIP: return "HIP kernel launch failed (see attn_last_hip_error)";
    default: return "unknown status";
  }
}

int attn_last_hip_error(void) { return g_last_hip_error; }

const char* attn_version(void) { return "attn 0.1.0 gfx950"; }

}  // extern "C"
