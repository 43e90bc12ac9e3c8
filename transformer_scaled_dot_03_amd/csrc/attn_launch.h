// Internal interface between the C-ABI entry points (attn_api.hip) and the
// kernels (attn_fwd_kernel.hip).  Not installed; the public ABI is attn.h.
#ifndef ATTN_LAUNCH_H_
#define ATTN_LAUNCH_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

enum class DType { BF16, F32 };

// Kernel arguments, passed by value.  Tensors are dense row-major
// [B, H, T, d]; the kernel derives every offset in 64-bit arithmetic.
struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const int32_t* key_lens;  // device [B] or nullptr (only read with key padding)
  float* lse;               // optional fp32 [B, H, Tq]: natural-log row normaliser (bf16 path)
  int B, H, Tq, Tk;
  float scale_log2;         // |scale| * log2(e): scores feed exp2
  int neg;                  // 1 when scale < 0: the kernel negates Q (exact)
  int n_qtiles;             // ceil(Tq / rows_per_block(dt, d))
  int n_wg;                 // B * H * n_qtiles work-groups
  // Element strides of batch entry, head and row for each tensor (the bf16
  // kernel honours them; the dense [B, H, T, d] layout has row = d, head = T d,
  // batch = H T d, and is what the fp32 kernel assumes).
  int64_t q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh;
  int q_sr, k_sr, v_sr, o_sr;
};
// fills the strides of the dense [B, H, T, d] layout
inline void set_dense_strides(Params& p, int d) {
  p.q_sr = p.k_sr = p.v_sr = p.o_sr = d;
  p.q_sh = p.o_sh = static_cast<int64_t>(p.Tq) * d;
  p.k_sh = p.v_sh = static_cast<int64_t>(p.Tk) * d;
  p.q_sb = p.o_sb = p.q_sh * p.H;
  p.k_sb = p.v_sb = p.k_sh * p.H;
}

// Backward pass arguments (bf16 tensors, fp32 lse and delta).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;         // [B, H, Tq] from the forward
  float* delta;             // [2, B, H, Tq] written by the dQ kernel: D_i = dO_i . O_i, then
                            // lse_i * log2(e) (+inf for a row with no allowed key)
  void* dq;
  void* dk;
  void* dv;
  const int32_t* key_lens;
  int B, H, Tq, Tk;
  float scale_log2;         // |scale| * log2(e) (>= 1e-30)
  float scale;              // the score scale (dQ = scale dS K, dK = scale dS^T Q)
  int neg;                  // 1 when scale < 0: the kernels negate Q (exact)
  int n_qtiles, n_ktiles;   // query / key tiles per (b, head)
};

// query rows per work-group of the kernel that serves (dt, d)
int rows_per_block(DType dt, int d);
hipError_t launch_fwd(const Params& p, DType dt, int d, bool causal, bool keypad, hipStream_t stream);

// Weights output: recompute the row softmax from the forward's log-sum-exp and
// store it as fp32 [B, H, Tq, Tk].
struct WtsParams {
  const void* q;
  const void* k;
  const float* lse;         // [B, H, Tq] from the forward
  float* w;                 // [B, H, Tq, Tk] written in full (zeros where masked)
  const int32_t* key_lens;
  int B, H, Tq, Tk;
  float scale_log2;
  int neg;
  int n_qtiles;
};
int weights_rows_per_block(int d);
hipError_t launch_weights(const WtsParams& p, int d, bool causal, bool keypad, hipStream_t stream);

// Projection GEMM of the multi-head wrapper: C[M x N] = A[M x K] B[K x N],
// bf16 operands and result, fp32 accumulation.  A is row-major [M x K], B is
// passed transposed (bt = B^T, row-major [N x K]), C row-major [M x N];
// leading dimensions in elements.  K a multiple of 64, N of 8; lda, ldb, ldc
// multiples of 8 (16-byte rows); pointers 16-byte aligned.
struct GemmParams {
  const void* a;
  const void* bt;
  void* c;
  int M, N, K;
  int lda, ldb, ldc;
  int n_mt, n_nt;           // row and column tiles of C (set by launch_gemm)
};
hipError_t launch_gemm(const GemmParams& p, hipStream_t stream);

// dst [C x R] = src [R x C]^T (bf16) for up to four matrices in one launch;
// R and C multiples of 64
struct TransposeJob {
  const __bf16* src;
  __bf16* dst;
};
struct TransposeJobs {
  TransposeJob job[4];
  int R, C;
};
hipError_t launch_transpose(const TransposeJobs& J, int njobs, hipStream_t stream);

// Multi-head attention forward (projection GEMMs, attention reading the
// projections in place through strides, output projection).  Workspace
// layout, byte offsets from its start.
struct MhaLayout {
  size_t wt;          // bf16 [4 d_model, d_model]: Wq^T, Wk^T, Wv^T, Wo^T (the GEMMs' B^T operands)
  size_t proj;        // bf16: [B T, 3 d_model] (self) or [B Tq, d_model] + [B Tk, 2 d_model] (cross)
  size_t o;           // bf16 [B, Tq, h, d]: the attention output, heads side by side
  size_t bytes;       // total
};
MhaLayout mha_layout(int B, int Tq, int Tk, int d_model);
struct MhaArgs {
  const void *xq, *xk, *xv;   // bf16 [B, Tq, dm], [B, Tk, dm], [B, Tk, dm]
  const void *wq, *wk, *wv;   // bf16 [dm, h d]
  const void* wo;             // bf16 [h d, dm]
  void* y;                    // bf16 [B, Tq, dm]
  void* workspace;
  int B, Tq, Tk, d_model, H, D;
  bool causal, keypad;
  bool fused_qkv;             // xq == xk == xv: one projection GEMM against [Wq | Wk | Wv]
  Params attn;                // scale, mask and tiling of the attention launch
};
// hipSuccess, or the first launch error
hipError_t mha_run(const MhaArgs& a, hipStream_t stream);

// Decode (one query row per (b, head)) split over the keys: arguments of the
// split kernel and of the merge kernel.
struct DecParams {
  const void* q;            // bf16 [B*H, d]
  const void* k;            // bf16 [B*H, Tk, d]
  const void* v;
  void* o;                  // bf16 [B*H, d]
  const int32_t* key_lens;  // device [B] or nullptr
  float* part_acc;          // fp32 [B*H, n_split, d]: unnormalised partial outputs
  float* part_ml;           // fp32 [B*H, n_split, 2]: partial (max, sum), log2 units
  int B, H, Tk;
  int keys_per_split;       // multiple of 256
  int n_split;
  float scale_log2;         // |scale| * log2(e) (>= 1e-30)
  int neg;                  // 1 when scale < 0: q is negated (exact)
};

// keys per split work-group and split count for a decode problem (the same
// function sizes the workspace and the launch)
int decode_keys_per_split(int B, int H, int Tk);
int decode_splits(int B, int H, int Tk);
hipError_t launch_decode(const DecParams& p, int d, bool keypad, hipStream_t stream);

// backward: query rows per dQ work-group and keys per dK/dV work-group
int bwd_rows_per_block(int d);
int bwd_keys_per_block(int d);
// enqueues the dQ kernel (which also writes delta), then the dK/dV kernel
hipError_t launch_bwd(const BwdParams& p, int d, bool causal, bool keypad, hipStream_t stream);

}  // namespace attn

#endif  // ATTN_LAUNCH_H_
