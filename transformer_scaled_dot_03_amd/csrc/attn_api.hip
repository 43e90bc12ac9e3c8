// C-ABI entry points of libattn.so (declared in include/attn.h).
//
// Host side only: argument validation (no HIP call is made before every
// check has passed), choice of the kernel instance and the launch on the
// caller's stream.  The operation itself is documented in attn.h.

#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "attn.h"
#include "attn_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

// Device scratch of attn_decode_static: one copy per GPU, held until the
// process ends.  In host code `scratch` names a host-side stand-in, never the
// device memory: kernels get the address hipGetSymbolAddress returns for the
// current device, looked up once per device and kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[ATTN_DECODE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
std::atomic<void*> g_scratch[kMaxDevices];
std::atomic<int> g_scratch_err[kMaxDevices];

// the device address of `scratch` on device `dev` (which must be current), or
// nullptr with the HIP error kept in g_last_hip_error
void* scratch_on_device(int dev) {
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e == hipSuccess && ptr != nullptr) g_scratch[dev].store(ptr, std::memory_order_release);
    else g_scratch_err[dev].store(e == hipSuccess ? static_cast<int>(hipErrorInvalidSymbol) : static_cast<int>(e),
                                  std::memory_order_release);
  });
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) g_last_hip_error = g_scratch_err[dev].load(std::memory_order_acquire);
  return ptr;
}

// byte ranges [a, a + na) and [b, b + nb); sizes in 128-bit so no product can wrap
bool overlaps(const void* a, unsigned __int128 na, const void* b, unsigned __int128 nb) {
  if (na == 0 || nb == 0) return false;
  const unsigned __int128 a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

// |scale| * log2(e), kept >= 1e-30 so that masked (-inf) scores always map to
// exp2(-inf) = 0; for scale = 0 every exp2 argument then rounds to 0 and the
// weights are exactly uniform, as for a true zero.
float scale_log2(float scale) {
  return static_cast<float>(std::fmax(std::fabs(static_cast<double>(scale)) * 1.4426950408889634, 1e-30));
}

int fwd(attn::DType dt, const void* q, const void* k, const void* v, void* out, float* lse, int B, int h,
        int Tq, int Tk, int d_k, int d_v, float scale, int mask_kind, const int32_t* key_lens,
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
  if (lse != nullptr && misaligned(lse, 4)) return ATTN_ERR_ALIGN;

  const int64_t bm = attn::rows_per_block(dt, d_k);
  const int64_t bh = static_cast<int64_t>(B) * h;
  const int64_t n_qtiles = (Tq + bm - 1) / bm;
  const int64_t n_wg = bh * n_qtiles;  // B, h < 2^31 and n_qtiles < 2^25: no overflow
  if (n_wg > 0x7fffffffLL) return ATTN_ERR_TOO_LARGE;
  // the kernels address one head's K / V rows through a buffer descriptor with a 32-bit byte range
  if (static_cast<int64_t>(Tk) * d_k * (dt == attn::DType::F32 ? 4 : 2) > 0xffffffffLL) return ATTN_ERR_TOO_LARGE;

  typedef unsigned __int128 u128;
  const u128 es = dt == attn::DType::F32 ? 4 : 2;
  const u128 nq = (u128)bh * Tq * d_k * es, nkv = (u128)bh * Tk * d_k * es, no = (u128)bh * Tq * d_v * es;
  const u128 nkl = keypad ? (u128)B * 4 : 0;   // key_lens is read by every work-group
  if (overlaps(out, no, q, nq) || overlaps(out, no, k, nkv) || overlaps(out, no, v, nkv) ||
      overlaps(out, no, key_lens, nkl))
    return ATTN_ERR_ALIAS;
  if (lse != nullptr) {
    const u128 nl = (u128)bh * Tq * 4;
    if (overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nkv) || overlaps(lse, nl, v, nkv) ||
        overlaps(lse, nl, out, no) || overlaps(lse, nl, key_lens, nkl))
      return ATTN_ERR_ALIAS;
  }

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
  p.scale_log2 = scale_log2(scale);
  p.neg = scale < 0.f ? 1 : 0;
  p.n_qtiles = static_cast<int>(n_qtiles);
  p.n_wg = static_cast<int>(n_wg);
  p.lse = lse;
  attn::set_dense_strides(p, d_k);
  const hipError_t e = attn::launch_fwd(p, dt, d_k, causal, keypad, stream);
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

int bwd(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
        float* delta, void* dq, void* dk, void* dv, int B, int h, int Tq, int Tk, int d_k, int d_v,
        float scale, int mask_kind, const int32_t* key_lens, hipStream_t stream) {
  if (B < 0 || h < 0 || Tq < 0 || Tk < 0 || d_k < 0 || d_v < 0) return ATTN_ERR_SHAPE;
  if (d_k != d_v) return ATTN_ERR_SHAPE;
  if (d_k != 64 && d_k != 128) return ATTN_ERR_HEADDIM;
  if (mask_kind & ~(ATTN_MASK_CAUSAL | ATTN_MASK_KEYPAD)) return ATTN_ERR_MASK;
  const bool causal = (mask_kind & ATTN_MASK_CAUSAL) != 0;
  const bool keypad = (mask_kind & ATTN_MASK_KEYPAD) != 0;
  if (keypad && key_lens == nullptr) return ATTN_ERR_MASK;
  if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
  if (B == 0 || h == 0 || (Tq == 0 && Tk == 0)) return ATTN_OK;  // nothing to write
  // pointers the launched kernels touch: Tq > 0 runs the dQ kernel (q, out,
  // dout, lse, delta, dq; k and v when Tk > 0), Tk > 0 the dK/dV kernel (k, v,
  // dk, dv; q, dout, lse, delta when Tq > 0)
  const bool rows = Tq > 0, keys = Tk > 0;
  if (rows && (q == nullptr || out == nullptr || dout == nullptr || lse == nullptr || delta == nullptr ||
               dq == nullptr))
    return ATTN_ERR_NULL;
  if (keys && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr)) return ATTN_ERR_NULL;
  if (rows && (misaligned(q, 16) || misaligned(out, 16) || misaligned(dout, 16) || misaligned(dq, 16) ||
               misaligned(lse, 4) || misaligned(delta, 4)))
    return ATTN_ERR_ALIGN;
  if (keys && (misaligned(k, 16) || misaligned(v, 16) || misaligned(dk, 16) || misaligned(dv, 16)))
    return ATTN_ERR_ALIGN;
  if (keypad && misaligned(key_lens, 4)) return ATTN_ERR_ALIGN;

  const int64_t bh = static_cast<int64_t>(B) * h;
  const int64_t bm = attn::bwd_rows_per_block(d_k), bn = attn::bwd_keys_per_block(d_k);
  const int64_t n_qtiles = (Tq + bm - 1) / bm, n_ktiles = (Tk + bn - 1) / bn;
  if (bh * n_qtiles > 0x7fffffffLL || bh * n_ktiles > 0x7fffffffLL) return ATTN_ERR_TOO_LARGE;
  // one head's rows (K, V in the dQ kernel; Q, dO in the dK/dV kernel) sit behind a 32-bit byte range
  if (static_cast<int64_t>(Tq > Tk ? Tq : Tk) * d_k * 2 > 0xffffffffLL) return ATTN_ERR_TOO_LARGE;

  // written: delta, dq (rows), dk, dv (keys); read: q, k, v, out, dout, lse
  typedef unsigned __int128 u128;
  const u128 nq = rows ? (u128)bh * Tq * d_k * 2 : 0, nkv = keys ? (u128)bh * Tk * d_k * 2 : 0;
  const u128 nr = rows ? (u128)bh * Tq * 4 : 0;   // lse; delta holds two such arrays
  const void* in_p[7] = {q, k, v, out, dout, lse, key_lens};
  const u128 in_n[7] = {nq, nkv, nkv, nq, nq, nr, keypad ? (u128)B * 4 : 0};
  const void* out_p[4] = {delta, dq, dk, dv};
  const u128 out_n[4] = {2 * nr, nq, nkv, nkv};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 7; ++j)
      if (overlaps(out_p[i], out_n[i], in_p[j], in_n[j])) return ATTN_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(out_p[i], out_n[i], out_p[j], out_n[j])) return ATTN_ERR_ALIAS;
  }

  attn::BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = out;
  p.dout = dout;
  p.lse = lse;
  p.delta = delta;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.key_lens = keypad ? key_lens : nullptr;
  p.B = B;
  p.H = h;
  p.Tq = Tq;
  p.Tk = Tk;
  p.scale_log2 = scale_log2(scale);
  p.scale = scale;
  p.neg = scale < 0.f ? 1 : 0;
  p.n_qtiles = static_cast<int>(n_qtiles);
  p.n_ktiles = static_cast<int>(n_ktiles);
  const hipError_t e = attn::launch_bwd(p, d_k, causal, keypad, stream);
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

int fwd_weights(const void* q, const void* k, const void* v, void* out, float* lse, float* weights, int B, int h,
                int Tq, int Tk, int d_k, int d_v, float scale, int mask_kind, const int32_t* key_lens,
                hipStream_t stream) {
  // the argument checks of the forward, in its order, before the weights' own
  if (B < 0 || h < 0 || Tq < 0 || Tk < 0 || d_k < 0 || d_v < 0 || d_k != d_v) return ATTN_ERR_SHAPE;
  if (d_k != 64 && d_k != 128) return ATTN_ERR_HEADDIM;
  if ((mask_kind & ~(ATTN_MASK_CAUSAL | ATTN_MASK_KEYPAD)) ||
      ((mask_kind & ATTN_MASK_KEYPAD) && key_lens == nullptr))
    return ATTN_ERR_MASK;
  if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
  if (B == 0 || h == 0 || Tq == 0) return ATTN_OK;
  if (lse == nullptr || (Tk > 0 && weights == nullptr)) return ATTN_ERR_NULL;
  if (weights != nullptr && misaligned(weights, 16)) return ATTN_ERR_ALIGN;
  {
    const int64_t bm = attn::weights_rows_per_block(d_k);
    if (static_cast<int64_t>(B) * h * ((Tq + bm - 1) / bm) > 0x7fffffffLL) return ATTN_ERR_TOO_LARGE;
  }
  if (Tk > 0) {
    typedef unsigned __int128 u128;
    const u128 bh = (u128)B * h;
    const u128 nw = bh * Tq * Tk * 4, nq = bh * Tq * d_k * 2, nkv = bh * Tk * d_k * 2, no = bh * Tq * d_v * 2;
    const u128 nl = bh * Tq * 4, nkl = (mask_kind & ATTN_MASK_KEYPAD) ? (u128)B * 4 : 0;
    if (overlaps(weights, nw, q, nq) || overlaps(weights, nw, k, nkv) || overlaps(weights, nw, v, nkv) ||
        overlaps(weights, nw, out, no) || overlaps(weights, nw, lse, nl) || overlaps(weights, nw, key_lens, nkl))
      return ATTN_ERR_ALIAS;
  }
  const int st = fwd(attn::DType::BF16, q, k, v, out, lse, B, h, Tq, Tk, d_k, d_v, scale, mask_kind, key_lens,
                     stream);
  if (st != ATTN_OK || B == 0 || h == 0 || Tq == 0 || Tk == 0) return st;
  const int64_t bm = attn::weights_rows_per_block(d_k);
  attn::WtsParams p;
  p.q = q;
  p.k = k;
  p.lse = lse;
  p.w = weights;
  p.key_lens = (mask_kind & ATTN_MASK_KEYPAD) ? key_lens : nullptr;
  p.B = B;
  p.H = h;
  p.Tq = Tq;
  p.Tk = Tk;
  p.scale_log2 = scale_log2(scale);
  p.neg = scale < 0.f ? 1 : 0;
  p.n_qtiles = static_cast<int>((Tq + bm - 1) / bm);
  const hipError_t e = attn::launch_weights(p, d_k, (mask_kind & ATTN_MASK_CAUSAL) != 0,
                                            (mask_kind & ATTN_MASK_KEYPAD) != 0, stream);
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

int mha_fwd(const void* xq, const void* xk, const void* xv, const void* wq, const void* wk, const void* wv,
            const void* wo, void* y, int B, int Tq, int Tk, int d_model, int h, float scale, int mask_kind,
            const int32_t* key_lens, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (B < 0 || Tq < 0 || Tk < 0 || d_model <= 0 || h <= 0 || d_model % h != 0) return ATTN_ERR_SHAPE;
  const int d = d_model / h;
  if (d != 64 && d != 128) return ATTN_ERR_HEADDIM;
  if (mask_kind & ~(ATTN_MASK_CAUSAL | ATTN_MASK_KEYPAD)) return ATTN_ERR_MASK;
  const bool causal = (mask_kind & ATTN_MASK_CAUSAL) != 0;
  const bool keypad = (mask_kind & ATTN_MASK_KEYPAD) != 0;
  if (keypad && key_lens == nullptr) return ATTN_ERR_MASK;
  if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
  if (B == 0 || Tq == 0) return ATTN_OK;
  const void* ptrs[6] = {xq, wq, wk, wv, wo, y};
  for (const void* p : ptrs)
    if (p == nullptr) return ATTN_ERR_NULL;
  if (Tk > 0 && (xk == nullptr || xv == nullptr)) return ATTN_ERR_NULL;
  if (workspace == nullptr) return ATTN_ERR_WORKSPACE;
  for (const void* p : ptrs)
    if (misaligned(p, 16)) return ATTN_ERR_ALIGN;
  if (misaligned(workspace, 256) || (Tk > 0 && (misaligned(xk, 16) || misaligned(xv, 16))))
    return ATTN_ERR_ALIGN;
  if (keypad && misaligned(key_lens, 4)) return ATTN_ERR_ALIGN;
  // the GEMMs take B T rows as a 32-bit count; one head's rows (stride up to
  // 3 d_model) sit behind a 32-bit buffer range in the attention kernel
  const int64_t tmax = Tq > Tk ? Tq : Tk;
  if (static_cast<int64_t>(B) * tmax > 0x7fffffffLL || tmax * 3 * d_model * 2 > 0xffffffffLL)
    return ATTN_ERR_TOO_LARGE;
  const int64_t bm = attn::rows_per_block(attn::DType::BF16, d);
  const int64_t n_qtiles = (Tq + bm - 1) / bm;
  if (static_cast<int64_t>(B) * h * n_qtiles > 0x7fffffffLL) return ATTN_ERR_TOO_LARGE;
  const attn::MhaLayout L = attn::mha_layout(B, Tq, Tk, d_model);
  if (workspace_bytes < L.bytes) return ATTN_ERR_WORKSPACE;

  typedef unsigned __int128 u128;
  const u128 row = (u128)d_model * 2, hw = (u128)d_model * d_model * 2;
  const u128 nxq = (u128)B * Tq * row, nxkv = (u128)B * Tk * row, ny = nxq, nw = L.bytes;
  const void* in_p[8] = {xq, xk, xv, wq, wk, wv, wo, key_lens};
  const u128 in_n[8] = {nxq, nxkv, nxkv, hw, hw, hw, hw, keypad ? (u128)B * 4 : 0};
  for (int j = 0; j < 8; ++j)
    if (overlaps(y, ny, in_p[j], in_n[j]) || overlaps(workspace, nw, in_p[j], in_n[j])) return ATTN_ERR_ALIAS;
  if (overlaps(y, ny, workspace, nw)) return ATTN_ERR_ALIAS;

  attn::MhaArgs a;
  a.xq = xq;
  a.xk = xk;
  a.xv = xv;
  a.wq = wq;
  a.wk = wk;
  a.wv = wv;
  a.wo = wo;
  a.y = y;
  a.workspace = workspace;
  a.B = B;
  a.Tq = Tq;
  a.Tk = Tk;
  a.d_model = d_model;
  a.H = h;
  a.D = d;
  a.causal = causal;
  a.keypad = keypad;
  a.fused_qkv = (xq == xk && xk == xv && Tq == Tk);
  attn::Params& p = a.attn;     // pointers and strides are set by mha_run for the chosen layout
  p.key_lens = keypad ? key_lens : nullptr;
  p.B = B;
  p.H = h;
  p.Tq = Tq;
  p.Tk = Tk;
  p.scale_log2 = scale_log2(scale);
  p.neg = scale < 0.f ? 1 : 0;
  p.n_qtiles = static_cast<int>(n_qtiles);
  p.n_wg = static_cast<int>(static_cast<int64_t>(B) * h * n_qtiles);
  p.lse = nullptr;
  const hipError_t e = attn::mha_run(a, stream);
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

// workspace layout of attn_decode: partial outputs, then partial (max, sum)
struct DecodeWorkspace {
  int n_split, keys_per_split;
  size_t acc_bytes, bytes;
};

DecodeWorkspace decode_workspace(int B, int h, int Tk, int d) {
  DecodeWorkspace w;
  w.keys_per_split = attn::decode_keys_per_split(B, h, Tk);
  w.n_split = attn::decode_splits(B, h, Tk);
  const size_t parts = static_cast<size_t>(B) * h * w.n_split;
  w.acc_bytes = (parts * d * 4 + 255) & ~static_cast<size_t>(255);
  w.bytes = w.acc_bytes + ((parts * 2 * 4 + 255) & ~static_cast<size_t>(255));
  return w;
}

// Argument checks of the decode entry points, in order, up to (not including)
// the workspace; `empty` is set for a valid no-op, `ws` to the workspace layout.
int decode_check(const void* q, const void* k, const void* v, const void* out, int B, int h, int Tk, int d_k,
                 int d_v, float scale, int mask_kind, const int32_t* key_lens, bool& empty, DecodeWorkspace& ws) {
  empty = false;
  if (B < 0 || h < 0 || Tk < 0 || d_k < 0 || d_v < 0) return ATTN_ERR_SHAPE;
  if (d_k != d_v) return ATTN_ERR_SHAPE;
  if (d_k != 64 && d_k != 128) return ATTN_ERR_HEADDIM;
  if (mask_kind & ~ATTN_MASK_KEYPAD) return ATTN_ERR_MASK;  // causal is not a decode mask
  const bool keypad = (mask_kind & ATTN_MASK_KEYPAD) != 0;
  if (keypad && key_lens == nullptr) return ATTN_ERR_MASK;
  if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
  if (B == 0 || h == 0) {
    empty = true;
    return ATTN_OK;
  }
  if (q == nullptr || out == nullptr) return ATTN_ERR_NULL;
  if (Tk > 0 && (k == nullptr || v == nullptr)) return ATTN_ERR_NULL;
  if (misaligned(q, 16) || misaligned(out, 16) || (Tk > 0 && (misaligned(k, 16) || misaligned(v, 16))))
    return ATTN_ERR_ALIGN;
  if (keypad && misaligned(key_lens, 4)) return ATTN_ERR_ALIGN;
  const int64_t bh = static_cast<int64_t>(B) * h;
  if (static_cast<int64_t>(Tk) * d_k * 2 > 0xffffffffLL) return ATTN_ERR_TOO_LARGE;
  ws = decode_workspace(B, h, Tk, d_k);
  if (bh * ws.n_split > 0x7fffffffLL || bh > 0x7fffffffLL) return ATTN_ERR_TOO_LARGE;
  typedef unsigned __int128 u128;
  const u128 nq = (u128)bh * d_k * 2, nkv = (u128)bh * Tk * d_k * 2;
  const u128 nkl = keypad ? (u128)B * 4 : 0;
  if (overlaps(out, nq, q, nq) || overlaps(out, nq, k, nkv) || overlaps(out, nq, v, nkv) ||
      overlaps(out, nq, key_lens, nkl))
    return ATTN_ERR_ALIAS;
  return ATTN_OK;
}

// enqueues the split and merge kernels with the partials in `workspace` (laid out as `ws`)
int decode_launch(const void* q, const void* k, const void* v, void* out, int B, int h, int Tk, int d_k,
                  float scale, int mask_kind, const int32_t* key_lens, void* workspace, const DecodeWorkspace& ws,
                  hipStream_t stream) {
  const bool keypad = (mask_kind & ATTN_MASK_KEYPAD) != 0;
  attn::DecParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = out;
  p.key_lens = keypad ? key_lens : nullptr;
  p.part_acc = static_cast<float*>(workspace);
  p.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + ws.acc_bytes);
  p.B = B;
  p.H = h;
  p.Tk = Tk;
  p.keys_per_split = ws.keys_per_split;
  p.n_split = ws.n_split;
  p.scale_log2 = scale_log2(scale);
  p.neg = scale < 0.f ? 1 : 0;
  const hipError_t e = attn::launch_decode(p, d_k, keypad, stream);
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

int decode(const void* q, const void* k, const void* v, void* out, int B, int h, int Tk, int d_k, int d_v,
           float scale, int mask_kind, const int32_t* key_lens, void* workspace, size_t workspace_bytes,
           hipStream_t stream) {
  bool empty = false;
  DecodeWorkspace ws{};
  const int st = decode_check(q, k, v, out, B, h, Tk, d_k, d_v, scale, mask_kind, key_lens, empty, ws);
  if (st != ATTN_OK || empty) return st;
  if (workspace == nullptr) return ATTN_ERR_WORKSPACE;
  if (misaligned(workspace, 16)) return ATTN_ERR_ALIGN;
  if (workspace_bytes < ws.bytes) return ATTN_ERR_WORKSPACE;
  typedef unsigned __int128 u128;
  const int64_t bh = static_cast<int64_t>(B) * h;
  const u128 nq = (u128)bh * d_k * 2, nkv = (u128)bh * Tk * d_k * 2, nw = ws.bytes;
  const u128 nkl = (mask_kind & ATTN_MASK_KEYPAD) ? (u128)B * 4 : 0;
  if (overlaps(workspace, nw, q, nq) || overlaps(workspace, nw, k, nkv) || overlaps(workspace, nw, v, nkv) ||
      overlaps(workspace, nw, out, nq) || overlaps(workspace, nw, key_lens, nkl))
    return ATTN_ERR_ALIAS;
  return decode_launch(q, k, v, out, B, h, Tk, d_k, scale, mask_kind, key_lens, workspace, ws, stream);
}

int decode_static(const void* q, const void* k, const void* v, void* out, int B, int h, int Tk, int d_k,
                  int d_v, float scale, int mask_kind, const int32_t* key_lens, hipStream_t stream) {
  bool empty = false;
  DecodeWorkspace ws{};
  const int st = decode_check(q, k, v, out, B, h, Tk, d_k, d_v, scale, mask_kind, key_lens, empty, ws);
  if (st != ATTN_OK || empty) return st;
  if (ws.bytes > ATTN_DECODE_STATIC_SCRATCH_BYTES) return ATTN_ERR_WORKSPACE;
  // the array is the current device's: the stream must run there
  int dev = -1, sdev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) {
    if (stream == nullptr) sdev = dev;   // the null stream runs on the current device
    else e = hipStreamGetDevice(stream, &sdev);
  }
  if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices || sdev != dev)) e = hipErrorInvalidDevice;
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return ATTN_ERR_HIP;
  }
  void* ws_ptr = scratch_on_device(dev);
  if (ws_ptr == nullptr) return ATTN_ERR_HIP;
  return decode_launch(q, k, v, out, B, h, Tk, d_k, scale, mask_kind, key_lens, ws_ptr, ws, stream);
}

}  // namespace

extern "C" {

size_t attn_mha_workspace_bytes(int B, int Tq, int Tk, int d_model) {
  if (B < 0 || Tq < 0 || Tk < 0 || d_model <= 0) return 0;
  return attn::mha_layout(B, Tq, Tk, d_model).bytes;
}

int attn_mha_fwd(const void* xq, const void* xk, const void* xv, const void* wq, const void* wk, const void* wv,
                 const void* wo, void* y, int B, int Tq, int Tk, int d_model, int h, float scale, int mask_kind,
                 const int32_t* key_lens, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return mha_fwd(xq, xk, xv, wq, wk, wv, wo, y, B, Tq, Tk, d_model, h, scale, mask_kind, key_lens, workspace,
                 workspace_bytes, stream);
}

int attn_fwd_weights(const void* q, const void* k, const void* v, void* out, float* lse, float* weights, int B,
                     int h, int Tq, int Tk, int d_k, int d_v, float scale, int mask_kind, const int32_t* key_lens,
                     hipStream_t stream) {
  return fwd_weights(q, k, v, out, lse, weights, B, h, Tq, Tk, d_k, d_v, scale, mask_kind, key_lens, stream);
}

int attn_decode_static(const void* q, const void* k, const void* v, void* out, int B, int h, int Tk, int d_k,
                       int d_v, float scale, int mask_kind, const int32_t* key_lens, hipStream_t stream) {
  return decode_static(q, k, v, out, B, h, Tk, d_k, d_v, scale, mask_kind, key_lens, stream);
}

size_t attn_decode_workspace_bytes(int B, int h, int Tk, int d) {
  if (B <= 0 || h <= 0 || Tk < 0 || (d != 64 && d != 128)) return 0;
  return decode_workspace(B, h, Tk, d).bytes;
}

int attn_decode(const void* q, const void* k, const void* v, void* out, int B, int h, int Tk, int d_k, int d_v,
                float scale, int mask_kind, const int32_t* key_lens, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
  return decode(q, k, v, out, B, h, Tk, d_k, d_v, scale, mask_kind, key_lens, workspace, workspace_bytes,
                stream);
}

int attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int h, int Tq, int Tk,
             int d_k, int d_v, float scale, int mask_kind, const int32_t* key_lens, hipStream_t stream) {
  return fwd(attn::DType::BF16, q, k, v, out, nullptr, B, h, Tq, Tk, d_k, d_v, scale, mask_kind, key_lens,
             stream);
}

int attn_fwd_lse(const void* q, const void* k, const void* v, void* out, float* lse, int B, int h, int Tq,
                 int Tk, int d_k, int d_v, float scale, int mask_kind, const int32_t* key_lens,
                 hipStream_t stream) {
  if (lse == nullptr && B > 0 && h > 0 && Tq > 0) return ATTN_ERR_NULL;
  return fwd(attn::DType::BF16, q, k, v, out, lse, B, h, Tq, Tk, d_k, d_v, scale, mask_kind, key_lens,
             stream);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
             float* delta, void* dq, void* dk, void* dv, int B, int h, int Tq, int Tk, int d_k, int d_v,
             float scale, int mask_kind, const int32_t* key_lens, hipStream_t stream) {
  return bwd(q, k, v, out, dout, lse, delta, dq, dk, dv, B, h, Tq, Tk, d_k, d_v, scale, mask_kind, key_lens,
             stream);
}

int attn_fwd_f32(const void* q, const void* k, const void* v, void* out, int B, int h, int Tq, int Tk,
                 int d_k, int d_v, float scale, int mask_kind, const int32_t* key_lens,
                 hipStream_t stream) {
  return fwd(attn::DType::F32, q, k, v, out, nullptr, B, h, Tq, Tk, d_k, d_v, scale, mask_kind, key_lens,
             stream);
}

const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer argument";
    case ATTN_ERR_SHAPE: return "bad shape (negative dimension or d_k != d_v)";
    case ATTN_ERR_HEADDIM: return "unsupported head size (supported: 64, 128)";
    case ATTN_ERR_MASK: return "bad mask_kind bits, or key padding without key_lens";
    case ATTN_ERR_ALIAS: return "an output overlaps an input or another output";
    case ATTN_ERR_ALIGN: return "misaligned pointer (bf16/fp32 tensors need 16 bytes; key_lens, lse, delta 4)";
    case ATTN_ERR_SCALE: return "scale is not finite";
    case ATTN_ERR_WORKSPACE:
      return "workspace missing or smaller than attn_decode_workspace_bytes() / attn_mha_workspace_bytes(), "
             "or (attn_decode_static) larger than ATTN_DECODE_STATIC_SCRATCH_BYTES";
    case ATTN_ERR_TOO_LARGE: return "too large: over 2^31-1 work-groups, or one head's rows of a tensor over 4 GiB";
    case ATTN_ERR_HIP: return "HIP kernel launch failed (see attn_last_hip_error)";
    default: return "unknown status";
  }
}

int attn_last_hip_error(void) { return g_last_hip_error; }

const char* attn_version(void) { return "attn 0.1.0 gfx950"; }

}  // extern "C"
