// Multi-head attention forward: MultiHead = Concat(head_1, ..., head_h) W^O,
// head_i = Attention(Xq W_i^Q, Xk W_i^K, Xv W_i^V) ("Attention Is All You Need"
// notebook chapter, "Multi-Head Self-Attention"; cuijiawei.cn MultiHeadAttention
// snippet: the projected rows viewed as [B, T, h, d], heads moved next to the
// batch, attention, then the inverse move and the output projection).  No bias
// terms: the formula has none.
//
// The projections are plain GEMMs and go to rocBLAS (bf16 operands, fp32
// accumulation, bf16 results); the attention is the fused kernel of
// attn_fwd_kernel.hip, which reads each head's rows straight out of the
// projected rows through (batch, head, row) strides and writes its output with
// the heads side by side, so no layout change is ever materialised:
//
//   self-attention (xq = xk = xv):  P = X [Wq | Wk | Wv]     [B T, 3 d_model]
//   otherwise:  P_q = Xq Wq [B Tq, d_model];  P_kv = [Xk Wk | Xv Wv] [B Tk, 2 d_model]
//   O = attention(head i: columns i d .. i d + d - 1)        [B, Tq, h, d]
//   Y = O Wo                                                  [B, Tq, d_model]
//
// Everything lives in the caller's workspace (see attn_mha_workspace_bytes);
// rocBLAS is pointed at a slice of it too.  The one rocBLAS handle per device
// is created on the first call on that device and kept for the process.

#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>
#include <stdint.h>

#include <mutex>

#include "attn_launch.h"

namespace attn {

// [Wq | Wk | Wv]: dst row r = (wq row r, wk row r, wv row r); 16 bytes per thread
constexpr int kCatThreads = 256;
__global__ __launch_bounds__(kCatThreads) void attn_concat3_kernel(const __bf16* __restrict__ w0,
                                                                  const __bf16* __restrict__ w1,
                                                                  const __bf16* __restrict__ w2,
                                                                  __bf16* __restrict__ dst, int rows, int cols) {
  const int c8 = cols / 8;
  const int64_t i = (int64_t)blockIdx.x * kCatThreads + threadIdx.x;   // over rows x 3 x c8, in dst order
  if (i >= (int64_t)rows * 3 * c8) return;
  const int c = (int)(i % c8);
  const int64_t rk = i / c8;
  const int k = (int)(rk % 3);
  const int64_t r = rk / 3;
  const __bf16* src = k == 0 ? w0 : (k == 1 ? w1 : w2);
  *reinterpret_cast<uint4*>(dst + i * 8) = *reinterpret_cast<const uint4*>(src + r * cols + 8 * c);
}

// ---------------------------------------------------------------------------
// rocBLAS: one handle per device, created on first use
// ---------------------------------------------------------------------------

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_blas_mutex;
rocblas_handle g_blas[kMaxDevices] = {};
}  // namespace

// row-major C[M x N] = A[M x K] B[K x N] with leading dimensions (elements) lda,
// ldb, ldc; bf16 operands and result, fp32 accumulation.  In rocBLAS'
// column-major terms this is C^T = B^T A^T with no transposes.
static rocblas_status gemm_rowmajor(rocblas_handle hd, int M, int N, int K, const void* A, int lda,
                                    const void* Bm, int ldb, void* C, int ldc) {
  const float one = 1.0f, zero = 0.0f;
  return rocblas_gemm_ex(hd, rocblas_operation_none, rocblas_operation_none, N, M, K, &one, Bm,
                         rocblas_datatype_bf16_r, ldb, A, rocblas_datatype_bf16_r, lda, &zero, C,
                         rocblas_datatype_bf16_r, ldc, C, rocblas_datatype_bf16_r, ldc, rocblas_datatype_f32_r,
                         rocblas_gemm_algo_standard, 0, 0);
}

MhaLayout mha_layout(int B, int Tq, int Tk, int d_model) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const size_t dm = static_cast<size_t>(d_model);
  MhaLayout l;
  l.wcat = 0;
  l.proj = l.wcat + up(3 * dm * dm * 2);
  l.o = l.proj + up(static_cast<size_t>(B) * (static_cast<size_t>(Tq) * dm + static_cast<size_t>(Tk) * 2 * dm) * 2);
  l.blas = l.o + up(static_cast<size_t>(B) * Tq * dm * 2);
  l.blas_bytes = kMhaBlasWorkspace;
  l.bytes = l.blas + l.blas_bytes;
  return l;
}

int mha_run(const MhaArgs& a, hipStream_t stream, int* blas_status, hipError_t* hip_status) {
  int dev = 0;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *hip_status = he != hipSuccess ? he : hipErrorInvalidDevice;
    return -1;
  }
  std::lock_guard<std::mutex> lock(g_blas_mutex);   // a rocBLAS handle serves one call at a time
  if (g_blas[dev] == nullptr) {
    rocblas_status st = rocblas_create_handle(&g_blas[dev]);
    if (st != rocblas_status_success) {
      g_blas[dev] = nullptr;
      *blas_status = static_cast<int>(st);
      return -2;
    }
  }
  rocblas_handle hd = g_blas[dev];
  char* ws = static_cast<char*>(a.workspace);
  const MhaLayout L = mha_layout(a.B, a.Tq, a.Tk, a.d_model);
  rocblas_status st = rocblas_set_stream(hd, stream);
  if (st == rocblas_status_success) st = rocblas_set_workspace(hd, ws + L.blas, L.blas_bytes);
  auto fail_blas = [&](rocblas_status s) {
    *blas_status = static_cast<int>(s);
    return -2;
  };
  auto fail_hip = [&](hipError_t e) {
    *hip_status = e;
    return -1;
  };
  if (st != rocblas_status_success) return fail_blas(st);

  const int dm = a.d_model, D = a.D;
  __bf16* proj = reinterpret_cast<__bf16*>(ws + L.proj);
  Params p = a.attn;
  if (a.fused_qkv) {
    // [Wq | Wk | Wv] side by side, then one GEMM: each projected row holds q, k, v of every head
    {
      const __bf16* w0 = static_cast<const __bf16*>(a.wq);
      const __bf16* w1 = static_cast<const __bf16*>(a.wk);
      const __bf16* w2 = static_cast<const __bf16*>(a.wv);
      __bf16* dst = reinterpret_cast<__bf16*>(ws + L.wcat);
      int rows = dm, cols = dm;
      void* args[] = {&w0, &w1, &w2, &dst, &rows, &cols};
      const int64_t n = static_cast<int64_t>(dm) * 3 * (dm / 8);
      he = hipLaunchKernel(reinterpret_cast<const void*>(&attn_concat3_kernel),
                           dim3(static_cast<unsigned>((n + kCatThreads - 1) / kCatThreads)), dim3(kCatThreads), args,
                           0, stream);
      if (he != hipSuccess) return fail_hip(he);
    }
    st = gemm_rowmajor(hd, a.B * a.Tq, 3 * dm, dm, a.xq, dm, ws + L.wcat, 3 * dm, proj, 3 * dm);
    if (st != rocblas_status_success) return fail_blas(st);
    p.q = proj;
    p.k = proj + dm;
    p.v = proj + 2 * dm;
    p.q_sr = p.k_sr = p.v_sr = 3 * dm;
    p.q_sb = p.k_sb = p.v_sb = static_cast<int64_t>(a.Tq) * 3 * dm;
  } else {
    // Q rows [B Tq, dm]; K and V rows interleaved in [B Tk, 2 dm]
    __bf16* pkv = proj + static_cast<size_t>(a.B) * a.Tq * dm;
    st = gemm_rowmajor(hd, a.B * a.Tq, dm, dm, a.xq, dm, a.wq, dm, proj, dm);
    if (st == rocblas_status_success && a.Tk > 0)
      st = gemm_rowmajor(hd, a.B * a.Tk, dm, dm, a.xk, dm, a.wk, dm, pkv, 2 * dm);
    if (st == rocblas_status_success && a.Tk > 0)
      st = gemm_rowmajor(hd, a.B * a.Tk, dm, dm, a.xv, dm, a.wv, dm, pkv + dm, 2 * dm);
    if (st != rocblas_status_success) return fail_blas(st);
    p.q = proj;
    p.k = pkv;
    p.v = pkv + dm;
    p.q_sr = dm;
    p.q_sb = static_cast<int64_t>(a.Tq) * dm;
    p.k_sr = p.v_sr = 2 * dm;
    p.k_sb = p.v_sb = static_cast<int64_t>(a.Tk) * 2 * dm;
  }
  // head i is columns i d .. i d + d - 1 of each projected row
  p.q_sh = p.k_sh = p.v_sh = D;
  // output heads side by side: [B, Tq, h, d] is the concatenation the last projection reads
  p.o = ws + L.o;
  p.o_sr = dm;
  p.o_sh = D;
  p.o_sb = static_cast<int64_t>(a.Tq) * dm;
  he = launch_fwd(p, DType::BF16, D, a.causal, a.keypad, stream);
  if (he != hipSuccess) return fail_hip(he);
  st = gemm_rowmajor(hd, a.B * a.Tq, dm, dm, ws + L.o, dm, a.wo, dm, a.y, dm);
  if (st != rocblas_status_success) return fail_blas(st);
  return 0;
}

}  // namespace attn
