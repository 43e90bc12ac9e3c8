// Multi-head attention forward: MultiHead = Concat(head_1, ..., head_h) W^O,
// head_i = Attention(Xq W_i^Q, Xk W_i^K, Xv W_i^V) ("Attention Is All You Need"
// notebook chapter, "Multi-Head Self-Attention"; cuijiawei.cn MultiHeadAttention
// snippet: the projected rows viewed as [B, T, h, d], heads moved next to the
// batch, attention, then the inverse move and the output projection).  No bias
// terms: the formula has none.
//
// The projections are plain GEMMs (attn_gemm_kernel.hip: bf16 operands, fp32
// accumulation, bf16 results) against the transposed weights, which one small
// kernel writes into the workspace first; the attention is the fused kernel of
// attn_fwd_kernel.hip, which reads each head's rows straight out of the
// projected rows through (batch, head, row) strides and writes its output with
// the heads side by side, so no layout change is ever materialised:
//
//   W^T = [Wq^T; Wk^T; Wv^T; Wo^T]                           [4 d_model, d_model]
//   self-attention (xq = xk = xv):  P = X [Wq | Wk | Wv]     [B T, 3 d_model]
//   otherwise:  P_q = Xq Wq [B Tq, d_model];  P_kv = [Xk Wk | Xv Wv] [B Tk, 2 d_model]
//   O = attention(head i: columns i d .. i d + d - 1)        [B, Tq, h, d]
//   Y = O Wo                                                  [B, Tq, d_model]
//
// Everything lives in the caller's workspace (see attn_mha_workspace_bytes);
// every step is a kernel launch on the caller's stream.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"

namespace attn {

MhaLayout mha_layout(int B, int Tq, int Tk, int d_model) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const size_t dm = static_cast<size_t>(d_model);
  MhaLayout l;
  l.wt = 0;
  l.proj = l.wt + up(4 * dm * dm * 2);
  l.o = l.proj + up(static_cast<size_t>(B) * (static_cast<size_t>(Tq) * dm + static_cast<size_t>(Tk) * 2 * dm) * 2);
  l.bytes = l.o + up(static_cast<size_t>(B) * Tq * dm * 2);
  return l;
}

// row-major C[M x N] = A[M x K] B[K x N], B given as B^T [N x K]; leading dimensions in elements
static hipError_t gemm(int M, int N, int K, const void* A, int lda, const void* Bt, int ldb, void* C, int ldc,
                       hipStream_t stream) {
  GemmParams g;
  g.a = A;
  g.bt = Bt;
  g.c = C;
  g.M = M;
  g.N = N;
  g.K = K;
  g.lda = lda;
  g.ldb = ldb;
  g.ldc = ldc;
  g.n_mt = g.n_nt = 0;
  return launch_gemm(g, stream);
}

hipError_t mha_run(const MhaArgs& a, hipStream_t stream) {
  char* ws = static_cast<char*>(a.workspace);
  const MhaLayout L = mha_layout(a.B, a.Tq, a.Tk, a.d_model);
  const int dm = a.d_model, D = a.D;
  __bf16* proj = reinterpret_cast<__bf16*>(ws + L.proj);
  // W^T of the four weights, one after the other: rows 0 .. 3 dm - 1 are
  // then [Wq | Wk | Wv]^T, the B^T of the fused projection
  __bf16* wt = reinterpret_cast<__bf16*>(ws + L.wt);
  const size_t dd = static_cast<size_t>(dm) * dm;
  TransposeJobs tj;
  const void* wsrc[4] = {a.wq, a.wk, a.wv, a.wo};
  for (int j = 0; j < 4; ++j) {
    tj.job[j].src = static_cast<const __bf16*>(wsrc[j]);
    tj.job[j].dst = wt + j * dd;
  }
  tj.R = tj.C = dm;
  hipError_t he = launch_transpose(tj, 4, stream);
  if (he != hipSuccess) return he;
  Params p = a.attn;
  if (a.fused_qkv) {
    // one GEMM: each projected row holds q, k, v of every head
    he = gemm(a.B * a.Tq, 3 * dm, dm, a.xq, dm, wt, dm, proj, 3 * dm, stream);
    if (he != hipSuccess) return he;
    p.q = proj;
    p.k = proj + dm;
    p.v = proj + 2 * dm;
    p.q_sr = p.k_sr = p.v_sr = 3 * dm;
    p.q_sb = p.k_sb = p.v_sb = static_cast<int64_t>(a.Tq) * 3 * dm;
  } else {
    // Q rows [B Tq, dm]; K and V rows interleaved in [B Tk, 2 dm]
    __bf16* pkv = proj + static_cast<size_t>(a.B) * a.Tq * dm;
    he = gemm(a.B * a.Tq, dm, dm, a.xq, dm, wt, dm, proj, dm, stream);
    if (he == hipSuccess && a.Tk > 0) he = gemm(a.B * a.Tk, dm, dm, a.xk, dm, wt + dd, dm, pkv, 2 * dm, stream);
    if (he == hipSuccess && a.Tk > 0) he = gemm(a.B * a.Tk, dm, dm, a.xv, dm, wt + 2 * dd, dm, pkv + dm, 2 * dm, stream);
    if (he != hipSuccess) return he;
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
  if (he != hipSuccess) return he;
  return gemm(a.B * a.Tq, dm, dm, ws + L.o, dm, wt + 3 * dd, dm, a.y, dm, stream);
}

}  // namespace attn
