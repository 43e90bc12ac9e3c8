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
  int B, H, Tq, Tk;
  float scale_log2;         // |scale| * log2(e): scores feed exp2
  int neg;                  // 1 when scale < 0: the kernel negates Q (exact)
  int n_qtiles;             // ceil(Tq / rows_per_block(dt, d))
  int n_wg;                 // B * H * n_qtiles work-groups
  float* lse;               // optional fp32 [B, H, Tq]: natural-log row normaliser (bf16 path)
};

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
