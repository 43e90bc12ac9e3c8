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
};

// query rows per work-group of the kernel that serves (dt, d)
int rows_per_block(DType dt, int d);
hipError_t launch_fwd(const Params& p, DType dt, int d, bool causal, bool keypad, hipStream_t stream);

}  // namespace attn

#endif  // ATTN_LAUNCH_H_
